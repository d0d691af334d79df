"""Throughput of the MXFP4 MoE layer (route + experts + combine) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole layer -- moe_route then moe_expert_mlp --
over one batch of synthetic tokens already resident in HBM.  The default
(headline) workload is the GPT-OSS-120B-shaped prefill with Zipf-biased
routing: T = 16384 tokens, d_model = d_ff = 2880, 128 experts, top-4, the
largest configuration of the benchmark set.  Expert weights are quantized to
MXFP4 once, outside the timed region (packed for the expert kernels), and
NCOPIES copies are rotated step to step so the 256 MB last-level cache cannot
hold them between steps.

Prints one JSON line.  `value` is tokens/s of the whole layer over K timed
steps.  `roofline` prices the dominant kernel (the gate/up expert kernel)
with its algorithmic work -- bytes for weight streaming, 4 D F flops per
routed pair for the grouped GEMM -- over its mean duration from HIP events
recorded on the layer's stream, against the published MI355X peak of what it
runs on (HBM 8 TB/s; fp4 x fp6 block-scaled matrix cores 10.1 PFLOP/s);
`roofline_down` does the same for the down kernel.  `traffic` is the HBM
bytes per launch from the committed rocprofv3 counter summary when it was
taken on the current kernel source, else null.  `cpu_baseline` is the
single-threaded fp64 CPU oracle on a bounded sample of the same workload.
With the headline workload (and without --no-configs) the line also carries
`configs`: the other four workloads and the headline's separately timed
mxfp4_quantize, each with its own timing and roofline, plus the two decode
workloads run again with bf16 expert weights (moe_expert_mlp_bf16, the
comparison path the pages name) with their weight-byte and time ratios to
the MXFP4 runs, and through moe_layer_decode (routing fused into the gate/up
weight stream) as `fused_decode`; and `probes`: the
achievable HBM read rate (also in the decode kernels' access order) and
matrix-core rates measured on this GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP6_PEAK_TFLOPS = 10100.0      # MI355X dense fp6 / fp4 matrix cores, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0       # dense fp8
F16_PEAK_TFLOPS = 2500.0       # dense fp16 / bf16
NCOPIES = 3
HEADLINE = "gptoss120b_prefill_skewed"
OTHER_CONFIGS = ["tiny", "gptoss20b_decode", "gptoss120b_decode", "gptoss20b_prefill"]
CONFIG_STEPS, CONFIG_WARMUP = 100, 10
# decode workloads also run with bf16 expert weights (the comparison path)
# and through the fused decode entry point
BF16_COMPARISON = ["gptoss20b_decode", "gptoss120b_decode"]
FUSED_DECODE = ["gptoss20b_decode", "gptoss120b_decode"]
ACT_TERMS = 3                  # grouped GEMM: x and h as 3 fp6 terms


def algorithmic_work(cfg, counts: np.ndarray) -> dict:
    """Bytes the layer must move and flops it must do (intermediates excluded)."""
    D, F, E, T, k = cfg.D, cfg.F, cfg.E, cfg.T, cfg.k
    touched = int((counts > 0).sum())
    w13_bytes = 2 * F * (D // 2 + D // 32)     # codes + E8M0 scales of one expert
    w2_bytes = D * (F // 2 + F // 32)
    x_bytes = 2 * T * D
    step_bytes = touched * (w13_bytes + w2_bytes) + 4 * E * D + 4 * E + x_bytes + 2 * T * D
    pairs = T * k
    return dict(touched=touched, step_bytes=step_bytes,
                gateup_bytes=touched * w13_bytes + x_bytes, down_bytes=touched * w2_bytes,
                step_flops=6 * D * F * pairs, gateup_flops=4 * D * F * pairs,
                down_flops=2 * D * F * pairs)


def packed_ok(cfg) -> bool:
    """Shapes the library accepts with packed weight codes (both expert
    algorithms: contraction sizes multiples of 64 within the streaming
    kernels' LDS budget)."""
    return cfg.D % 64 == 0 and cfg.F % 64 == 0 and cfg.D <= 3840 and cfg.F <= 2944


def uses_grouped_gemm(cfg, algo: str) -> bool:
    """The library's automatic choice: the grouped GEMM once the average expert
    receives 32 pairs, weight streaming below that."""
    return algo == "gemm" or (algo == "auto" and cfg.T * cfg.k >= 32 * cfg.E)


def kernel_source_digest(source: str) -> str:
    """sha256 over a kernel's source file followed by every device header of
    the library (sorted by name): the code a kernel is built from."""
    csrc = os.path.join(ROOT, "mxfp4_quantized_mixture_amd", "csrc")
    h = hashlib.sha256()
    for name in [source] + sorted(f for f in os.listdir(csrc) if f.endswith(".h")):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def read_traffic(kernel: str, workload: str, source: str, layout: str):
    """HBM bytes per dispatch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source (kernel_source_digest) with the same
    weight layout (else None)."""
    path = os.path.join(ROOT, "profiles", "%s.%s.traffic.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    digest = kernel_source_digest(source)
    if fields.get("kernel_source_sha256") != digest or fields.get("weight_layout") != layout:
        return None
    try:
        return float(fields["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def host_cpu() -> dict:
    model = "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        nproc = int(subprocess.run(["nproc"], capture_output=True, text=True,
                                   timeout=20).stdout.strip())
    except (OSError, subprocess.SubprocessError, ValueError):
        nproc = os.cpu_count()
    return {"model": model, "nproc": nproc}


def cpu_baseline(cfg, inp, sample_tokens: int = 32) -> dict:
    """The CPU oracle as it is (single-threaded C, fp64) on a bounded sample of
    the same workload, in tokens/s.  Routing runs for all T tokens; the expert
    MLP and combine for all tokens when T <= 64, else for `sample_tokens`
    evenly spaced tokens.  The oracle decodes each expert's weights once per
    call (a fixed cost a per expert, measured on its own) and then spends
    about b per routed pair, so the whole-workload time is extrapolated as
    t_route + (touched experts) a + T k b, with b taken from the sample."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle as orc

    x, wr, b, w13, w2 = inp
    T, k, E = cfg.T, cfg.k, cfg.E
    t0 = time.perf_counter()
    r = orc.route(x, wr, b, k)
    t_route = time.perf_counter() - t0
    tokens = np.arange(T) if T <= 64 else np.arange(0, T, T // sample_tokens)[:sample_tokens]
    used = sorted(set(r["ids"][tokens].ravel().tolist()))
    # quantizing the weights for the oracle is input preparation: untimed
    q13 = np.zeros((E, 2 * cfg.F, cfg.D // 2), np.uint8)
    s13 = np.zeros((E, 2 * cfg.F, cfg.D // 32), np.uint8)
    q2 = np.zeros((E, cfg.D, cfg.F // 2), np.uint8)
    s2 = np.zeros((E, cfg.D, cfg.F // 32), np.uint8)

    def prep(e):
        q13[e], s13[e] = orc.quantize(w13[e])
        q2[e], s2[e] = orc.quantize(w2[e])

    with ThreadPoolExecutor(max_workers=16) as ex:
        list(ex.map(prep, used))
    t0 = time.perf_counter()
    orc.moe(x, q13, s13, q2, s2, r["ids"], r["w"], cfg.F,
            tokens=None if T <= 64 else tokens.astype(np.int32))
    t_moe = time.perf_counter() - t0
    touched = int(len(np.unique(r["ids"])))
    if T <= 64:
        secs = t_route + t_moe
        how = "whole workload: route, %d experts' MLPs for all %d pairs, combine" % (
            touched, T * k)
        sample = "all %d tokens" % T
    else:
        e0 = used[0]
        t0 = time.perf_counter()
        orc.expert_mlp(x, q13[e0], s13[e0], q2[e0], s2[e0], cfg.F, np.zeros(0, np.int32))
        a = time.perf_counter() - t0
        pairs = len(tokens) * k
        bpair = max(t_moe - len(used) * a, 0.0) / pairs
        secs = t_route + touched * a + T * k * bpair
        how = ("route over all %d tokens (%.1f s); expert MLP + combine for %d tokens "
               "(%d pairs on %d experts, %.1f s); per-expert weight decode a = %.2f s, per "
               "pair b = %.1f ms; whole workload = route + %d a + %d b" %
               (T, t_route, len(tokens), pairs, len(used), t_moe, a, bpair * 1e3, touched,
                T * k))
        sample = "every %d-th token: %d of %d" % (T // sample_tokens, len(tokens), T)
    return {"value": T / secs, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": sample, "method": how, "seconds_measured": t_route + t_moe,
            "seconds_whole_workload": secs, "host_cpu": host_cpu()}


def bf16_dev(torch, dev, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def time_layers(layers, steps, warmup, moe, torch):
    """Warm up, then time `steps` steps rotating over the prepared layers
    (the weight copies): region 1 (the `value` region) with nothing but the
    layer on the stream, region 2 with HIP events recorded on the layer's
    stream around each expert kernel.  Returns (total ms of region 1, mean
    per-stage ms of region 2)."""
    n = len(layers)
    torch.cuda.synchronize()
    for i in range(warmup):
        layers[i % n]()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        layers[i % n]()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    evarr = [moe.PreparedLayer.event_array(e) for e in ev]
    torch.cuda.synchronize()
    for i in range(steps):
        layers[i % n](evarr[i])
    torch.cuda.synchronize()
    stage = {"gate_up": float(np.mean([e[0].elapsed_time(e[1]) for e in ev])),
             "down": float(np.mean([e[1].elapsed_time(e[2]) for e in ev])),
             "combine": float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))}
    return total_ms, stage


def run_layer(cfg, steps, warmup, seed, algo, layout, moe, torch, dev, keep_inputs=False):
    """Quantize, time `steps` layer steps (value region, then a second region
    with per-stage events) and return timings plus what the rooflines need."""
    from synth import moe_inputs as MI

    wr, b = MI.gen_router(cfg, seed)
    x = MI.gen_x(cfg, seed)
    w13, w2 = MI.gen_experts(cfg, seed, threads=16)
    xd, wrd, bd = bf16_dev(torch, dev, x), torch.from_numpy(wr).to(dev), torch.from_numpy(b).to(dev)
    packed = layout == "packed" or (layout == "auto" and packed_ok(cfg))
    w13d, w2d = bf16_dev(torch, dev, w13), bf16_dev(torch, dev, w2)
    base = moe.ExpertWeights.quantize(w13d, w2d, packed=packed)
    if not keep_inputs:
        del w13d, w2d
    copies = [base] + [moe.ExpertWeights(base.w13_q.clone(), base.w13_s.clone(),
                                         base.w2_q.clone(), base.w2_s.clone(), packed)
                       for _ in range(NCOPIES - 1)]
    out = torch.empty(cfg.T, cfg.D, dtype=torch.bfloat16, device=dev)
    routing = moe.alloc_routing(cfg.T, cfg.E, cfg.k, dev)
    route_ws = moe.route_workspace(cfg.T, cfg.D, cfg.E, cfg.k, dev)
    mlp_ws = moe.mlp_workspace(cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, dev)
    algo_id = {"auto": moe.MLP_AUTO, "stream": moe.MLP_STREAM, "gemm": moe.MLP_GROUPED_GEMM}[algo]
    layers = [moe.PreparedLayer(xd, wrd, bd, w, cfg.k, out, routing, route_ws, mlp_ws, algo=algo_id)
              for w in copies]
    total_ms, stage = time_layers(layers, steps, warmup, moe, torch)
    res = dict(ms_per_step=total_ms / steps, stage_ms=stage, counts=routing.counts.cpu().numpy(),
               packed=packed, gemm=uses_grouped_gemm(cfg, algo))
    if keep_inputs:
        res["inputs"] = (x, wr, b, w13, w2)
        res["bf16_weights"] = (w13d, w2d)
    del layers, copies, base, mlp_ws, route_ws
    torch.cuda.synchronize()
    return res


def run_layer_bf16(cfg, steps, warmup, seed, moe, torch, dev):
    """The same layer with bf16 expert weights (moe_expert_mlp_bf16, the
    comparison path): same inputs, routing and timing protocol as run_layer,
    NCOPIES weight copies rotated.  Returns timings and HBM rooflines of its
    two expert kernels, priced with the bf16 weight bytes."""
    from synth import moe_inputs as MI

    wr, b = MI.gen_router(cfg, seed)
    x = MI.gen_x(cfg, seed)
    w13, w2 = MI.gen_experts(cfg, seed, threads=16)
    xd, wrd, bd = bf16_dev(torch, dev, x), torch.from_numpy(wr).to(dev), torch.from_numpy(b).to(dev)
    base = (bf16_dev(torch, dev, w13), bf16_dev(torch, dev, w2))
    del w13, w2
    copies = [base] + [(base[0].clone(), base[1].clone()) for _ in range(NCOPIES - 1)]
    out = torch.empty(cfg.T, cfg.D, dtype=torch.bfloat16, device=dev)
    routing = moe.alloc_routing(cfg.T, cfg.E, cfg.k, dev)
    route_ws = moe.route_workspace(cfg.T, cfg.D, cfg.E, cfg.k, dev)
    mlp_ws = moe.mlp_bf16_workspace(cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, dev)
    layers = [moe.PreparedLayer(xd, wrd, bd, w, cfg.k, out, routing, route_ws, mlp_ws)
              for w in copies]
    total_ms, st = time_layers(layers, steps, warmup, moe, torch)
    counts = routing.counts.cpu().numpy()
    del layers, copies, base, mlp_ws, route_ws
    torch.cuda.synchronize()
    touched = int((counts > 0).sum())
    D, F = cfg.D, cfg.F
    gu_bytes = touched * 2 * F * D * 2 + 2 * cfg.T * D
    dn_bytes = touched * D * F * 2

    def hbm(bytes_, ms, kernel, traffic):
        a = bytes_ / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": a / HBM_PEAK_GBS, "traffic": traffic, "kernel": kernel,
                "algorithmic_per_launch": bytes_, "avg_launch_ms": ms}

    ms = total_ms / steps
    return {"workload": cfg.description + ", bf16 expert weights", "expert_weights": "bf16",
            "tokens_per_s": cfg.T / (ms * 1e-3), "ms_per_step": ms, "steps": steps,
            "warmup": warmup, "stage_ms": st, "touched_experts": touched,
            "roofline": hbm(gu_bytes, st["gate_up"], "expert_bf16_kernel<gate_up>",
                            read_traffic("gateup_bf16", cfg.name, "expert_bf16.hip", "bf16")),
            "roofline_down": hbm(dn_bytes, st["down"], "expert_bf16_kernel<down>",
                                 read_traffic("down_bf16", cfg.name, "expert_bf16.hip", "bf16"))}


def run_layer_fused_decode(cfg, steps, warmup, seed, moe, torch, dev):
    """The same decode step through moe_layer_decode (routing fused into the
    gate/up weight stream; packed codes): same inputs and timing protocol as
    run_layer, NCOPIES weight copies rotated."""
    from synth import moe_inputs as MI

    wr, b = MI.gen_router(cfg, seed)
    x = MI.gen_x(cfg, seed)
    w13, w2 = MI.gen_experts(cfg, seed, threads=16)
    xd, wrd, bd = bf16_dev(torch, dev, x), torch.from_numpy(wr).to(dev), torch.from_numpy(b).to(dev)
    base = moe.ExpertWeights.quantize(bf16_dev(torch, dev, w13), bf16_dev(torch, dev, w2),
                                      packed=True)
    del w13, w2
    copies = [base] + [moe.ExpertWeights(base.w13_q.clone(), base.w13_s.clone(),
                                         base.w2_q.clone(), base.w2_s.clone(), True)
                       for _ in range(NCOPIES - 1)]
    out = torch.empty(cfg.T, cfg.D, dtype=torch.bfloat16, device=dev)
    routing = moe.alloc_routing(cfg.T, cfg.E, cfg.k, dev)
    ws = moe.decode_workspace(cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, dev)
    layers = [moe.PreparedDecodeLayer(xd, wrd, bd, w, cfg.k, out, routing, ws) for w in copies]
    total_ms, st = time_layers(layers, steps, warmup, moe, torch)
    err = moe.decode_error(ws)
    del layers, copies, base, ws
    torch.cuda.synchronize()
    ms = total_ms / steps
    return {"entry_point": "moe_layer_decode", "tokens_per_s": cfg.T / (ms * 1e-3),
            "ms_per_step": ms, "steps": steps, "warmup": warmup,
            "stage_ms": {"route_and_gate_up": st["gate_up"], "down": st["down"],
                         "combine": st["combine"]},
            "device_wait_errors": err}


def bf16_comparison(cfg, mx, bf) -> dict:
    """Weight bytes and times of the bf16 path relative to the MXFP4 one."""
    w_mx = mx["roofline"]["algorithmic_per_launch"] - 2 * cfg.T * cfg.D
    w_bf = bf["roofline"]["algorithmic_per_launch"] - 2 * cfg.T * cfg.D
    return {"gate_up_weight_bytes_ratio": w_bf / w_mx,
            "gate_up_time_ratio": bf["stage_ms"]["gate_up"] / mx["stage_ms"]["gate_up"],
            "down_time_ratio": bf["stage_ms"]["down"] / mx["stage_ms"]["down"],
            "step_time_ratio": bf["ms_per_step"] / mx["ms_per_step"]}


def rooflines(cfg, run) -> tuple[dict, dict, dict]:
    """(gate/up kernel, down kernel, whole layer) rooflines."""
    work = algorithmic_work(cfg, run["counts"])
    st, gemm, packed = run["stage_ms"], run["gemm"], run["packed"]
    layout = "packed" if packed else "row-major"
    kinds = ",packed" if packed else ""
    if not gemm:
        def hbm(bytes_, ms, kernel, traffic):
            a = bytes_ / (ms * 1e-3) / 1e9
            return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": a / HBM_PEAK_GBS, "traffic": traffic, "kernel": kernel,
                    "algorithmic_per_launch": bytes_, "avg_launch_ms": ms}
        gu = hbm(work["gateup_bytes"], st["gate_up"], "expert_stream_kernel<gate_up%s>" % kinds,
                 read_traffic("gateup", cfg.name, "expert_mlp.hip", layout))
        dn = hbm(work["down_bytes"], st["down"], "expert_stream_kernel<down%s>" % kinds,
                 read_traffic("down", cfg.name, "expert_mlp.hip", layout))
        a = work["step_bytes"] / (run["ms_per_step"] * 1e-3) / 1e9
        layer = {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": a / HBM_PEAK_GBS}
    else:
        def mfma(flops, ms, kernel, traffic):
            a = flops / (ms * 1e-3) / 1e12
            # the activations enter as ACT_TERMS fp6 terms: the matrix cores
            # execute ACT_TERMS times the algorithmic flops
            return {"bound": "mfma", "achieved": a, "peak": FP6_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": a / FP6_PEAK_TFLOPS, "traffic": traffic, "kernel": kernel,
                    "algorithmic_per_launch": flops, "avg_launch_ms": ms,
                    "operand_types": "fp4 (E2M1) weights x fp6 (E2M3) activation terms",
                    "executed_tflops": ACT_TERMS * a,
                    "executed_frac": ACT_TERMS * a / FP6_PEAK_TFLOPS}
        gu = mfma(work["gateup_flops"], st["gate_up"], "expert_gemm_kernel<gate_up%s>" % kinds,
                  read_traffic("gateup_gemm", cfg.name, "expert_gemm.hip", layout))
        dn = mfma(work["down_flops"], st["down"], "expert_gemm_kernel<down%s>" % kinds,
                  read_traffic("down_gemm", cfg.name, "expert_gemm.hip", layout))
        a = work["step_flops"] / (run["ms_per_step"] * 1e-3) / 1e12
        layer = {"bound": "mfma", "achieved": a, "peak": FP6_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": a / FP6_PEAK_TFLOPS, "executed_frac": ACT_TERMS * a / FP6_PEAK_TFLOPS}
    layer["touched_experts"] = work["touched"]
    return gu, dn, layer


def quantize_timing(mats, steps, moe, torch) -> dict:
    """mxfp4_quantize of the given bf16 matrices (one call each per step),
    nearest-even and stochastic rounding; HBM bytes = 2 B read per element +
    0.5 + 1/32 B written."""
    elems = sum(m.numel() for m in mats)
    nbytes = elems * 2 + elems // 2 + elems // 32
    out = {"bytes_per_step": nbytes, "matrices": [list(m.shape) for m in mats]}
    for name, kw in (("nearest_even", {}), ("stochastic", {"stochastic": True, "seed": 1})):
        rule = moe.SCALE_CEIL_DIV6 if kw else moe.SCALE_FLOOR_DIV6
        for _ in range(2):
            for m in mats:
                moe.mxfp4_quantize(m, rule, **kw)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            for m in mats:
                moe.mxfp4_quantize(m, rule, **kw)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / steps
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "achieved_GBs": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
                     "steps": steps}
    return out


def probes(torch, dev) -> dict:
    """Achievable ceilings on this GPU (libmoe_probe.so): one streaming read of
    a 4 GiB buffer (far beyond the 256 MB last-level cache), the decode
    kernels' byte counts read in a private range per wavefront and as a
    grid-wide sweep, and 8 independent 32x32 matrix-core chains per wavefront
    for each operand type."""
    import ctypes

    from mxfp4_quantized_mixture_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        raise ImportError("%s is not built (python -m mxfp4_quantized_mixture_amd.build)"
                          % B.PROBE_LIB)
    L = ctypes.CDLL(B.PROBE_LIB)
    P = ctypes.c_void_p
    L.moe_probe_read.argtypes = [P, ctypes.c_size_t, ctypes.c_int, P, P]
    L.moe_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    L.moe_probe_mfma_flops.argtypes = [ctypes.c_int]
    L.moe_probe_mfma_flops.restype = ctypes.c_double
    stream = torch.cuda.current_stream(dev).cuda_stream
    res = {}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    for blocks in (2048, 8192):
        sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
        for _ in range(2):
            assert L.moe_probe_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), stream) == 0
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(5):
            L.moe_probe_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), stream)
        stop.record()
        torch.cuda.synchronize()
        res["hbm_read_GBs_%d_blocks" % blocks] = 5 * nbytes / (start.elapsed_time(stop) * 1e-3) / 1e9
    del buf
    # About the decode streaming kernels' byte counts (142, 283 and 508 MB),
    # read by 2048 wavefronts in two orders: each wavefront a private
    # contiguous range (as a wavefront owning whole weight tiles reads), and
    # the grid sweeping the buffer together.  Buffers rotate over more than
    # 1.5 GB so that no repeat finds its bytes in the 256 MB last-level cache;
    # the median of 20 single launches, each between two events.
    L.moe_probe_read_grouped.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    blocks = 256
    sink = torch.empty(blocks * 512, dtype=torch.int32, device=dev)
    rows = []
    for cpw in (68, 135, 242):
        nbytes = blocks * 8 * cpw * 1024
        nbuf = max(3, (1536 << 20) // nbytes + 1)
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        row = {"bytes": nbytes}
        for name, group in (("private", 1), ("sweep", blocks * 8)):
            for b in bufs:
                assert L.moe_probe_read_grouped(b.data_ptr(), cpw, blocks, group,
                                                sink.data_ptr(), stream) == 0
            times = []
            for r in range(20):
                start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                start.record()
                L.moe_probe_read_grouped(bufs[r % nbuf].data_ptr(), cpw, blocks, group,
                                         sink.data_ptr(), stream)
                stop.record()
                torch.cuda.synchronize()
                times.append(start.elapsed_time(stop))
            times.sort()
            row[name + "_us"] = times[len(times) // 2] * 1e3
            row[name + "_GBs"] = nbytes / (times[len(times) // 2] * 1e-3) / 1e9
        rows.append(row)
        del bufs
    res["read_patterns_2048_waves"] = rows
    names = {0: "fp4_fp4", 1: "fp4_fp6", 2: "fp4_fp8", 3: "fp8_fp8", 4: "f16", 5: "bf16"}
    blocks, iters = 2048, 500
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    for kind, name in names.items():
        assert L.moe_probe_mfma(kind, blocks, 10, sink.data_ptr(), stream) == 0
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        L.moe_probe_mfma(kind, blocks, iters, sink.data_ptr(), stream)
        stop.record()
        torch.cuda.synchronize()
        flops = blocks * 4 * 8 * iters * L.moe_probe_mfma_flops(kind)
        res["mfma_TFLOPs_" + name] = flops / (start.elapsed_time(stop) * 1e-3) / 1e12
    res["published_peaks"] = {"hbm_GBs": HBM_PEAK_GBS, "fp4_fp6_TFLOPs": FP6_PEAK_TFLOPS,
                              "fp8_TFLOPs": FP8_PEAK_TFLOPS, "f16_bf16_TFLOPs": F16_PEAK_TFLOPS}
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="only the named workload: no per-config results, quantize timing or probes")
    ap.add_argument("--algo", default="auto", choices=["auto", "stream", "gemm"],
                    help="expert algorithm (default: the library's automatic choice)")
    ap.add_argument("--layout", default="auto", choices=["auto", "canonical", "packed"],
                    help="expert weight code layout (default: packed where the kernels take it)")
    ap.add_argument("--quantize", action="store_true",
                    help="only time mxfp4_quantize (nearest-even and stochastic rounding) on the "
                         "workload's expert weights (W13 and W2)")
    ap.add_argument("--probes", action="store_true",
                    help="only run the achievable-peak probes (HBM reads, matrix cores)")
    ap.add_argument("--fused-decode", action="store_true",
                    help="only run the workload through moe_layer_decode (routing fused into "
                         "the gate/up weight stream; decode-sized workloads)")
    ap.add_argument("--bf16-weights", action="store_true",
                    help="only run the bf16-weight comparison path (moe_expert_mlp_bf16) on the "
                         "workload")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (calibrates "
                         "the HBM byte counters against a kernel of known traffic)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer here is the single-GPU hot path "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import mxfp4_quantized_mixture_amd as moe
    from synth import moe_inputs as MI

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        nbytes = 1 << 30
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": nbytes, "dispatches": 5}), flush=True)
        return 0
    if args.probes:
        print(json.dumps({"probes": probes(torch, dev)}), flush=True)
        return 0
    cfg = MI.CONFIGS[args.workload]
    if args.quantize:
        w13, w2 = MI.gen_experts(cfg, args.seed, threads=16)
        mats = [bf16_dev(torch, dev, a.reshape(-1, a.shape[-1])) for a in (w13, w2)]
        q = quantize_timing(mats, max(args.steps // 20, 5), moe, torch)
        print(json.dumps({"metric": "mxfp4_quantize HBM GB/s",
                          "workload": "%s: all %d experts' W13 and W2" % (cfg.name, cfg.E),
                          "results": q}), flush=True)
        return 0

    if args.fused_decode:
        r = run_layer_fused_decode(cfg, args.steps, args.warmup, args.seed, moe, torch, dev)
        print(json.dumps({"metric": "MXFP4 MoE-layer tokens/s, fused decode entry point",
                          "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                          "config": {"workload": cfg.description, "name": cfg.name},
                          "fused_decode": r}), flush=True)
        return 0
    if args.bf16_weights:
        r = run_layer_bf16(cfg, args.steps, args.warmup, args.seed, moe, torch, dev)
        print(json.dumps({"metric": "MXFP4 MoE-layer tokens/s, bf16-weight comparison path",
                          "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                          "config": {"workload": cfg.description, "name": cfg.name},
                          "bf16_weights": r}), flush=True)
        return 0

    headline = args.workload == HEADLINE and not args.no_configs
    run = run_layer(cfg, args.steps, args.warmup, args.seed, args.algo, args.layout, moe, torch,
                    dev, keep_inputs=headline or not args.no_cpu_baseline)
    gu, dn, layer = rooflines(cfg, run)
    ms = run["ms_per_step"]
    result = {
        "metric": "MXFP4 MoE-layer tokens/s",
        "value": cfg.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp4 x fp6 terms -> f32" if run["gemm"] else "mxfp4 x fp8 terms -> f32"),
        "data": "synthetic",
        "config": {"workload": cfg.description, "name": cfg.name, "tokens": cfg.T,
                   "d_model": cfg.D, "d_ff": cfg.F, "experts": cfg.E, "top_k": cfg.k,
                   "expert_weights": "mxfp4 (e2m1 + e8m0 per 32)",
                   "matrix_cores": ("block-scaled mfma: mxfp4 weights as stored x x and h as 3 "
                                    "fp6 (e2m3) terms, fp32 accumulate") if run["gemm"] else
                                   ("block-scaled mfma: mxfp4 weights as stored x x as 2 and h as "
                                    "3 fp8 (e4m3) terms, fp32 accumulate"),
                   "expert_algorithm": "grouped gemm" if run["gemm"] else "weight streaming",
                   "weight_layout": "packed 32x64 fragments" if run["packed"] else "row-major",
                   "touched_experts": layer["touched_experts"], "weight_copies_rotated": NCOPIES,
                   "parallelism": "single GPU"},
        "roofline": gu,
        "roofline_down": dn,
        "layer_roofline": layer,
        "stage_ms": run["stage_ms"],
    }
    if headline:
        w13d, w2d = run.pop("bf16_weights")
        mats = [w13d.view(-1, w13d.shape[-1]), w2d.view(-1, w2d.shape[-1])]
        q = quantize_timing(mats, 10, moe, torch)
        q["workload"] = "%s: all %d experts' W13 [%d, %d] and W2 [%d, %d] bf16" % (
            cfg.name, cfg.E, cfg.E * 2 * cfg.F, cfg.D, cfg.E * cfg.D, cfg.F)
        del mats, w13d, w2d
        torch.cuda.synchronize()
        configs = {"quantize_" + cfg.name: q}
        for name in OTHER_CONFIGS:
            c = MI.CONFIGS[name]
            r = run_layer(c, CONFIG_STEPS, CONFIG_WARMUP, args.seed, "auto", "auto", moe, torch,
                          dev)
            g2, d2, l2 = rooflines(c, r)
            configs[name] = {"workload": c.description, "tokens_per_s": c.T / (r["ms_per_step"] * 1e-3),
                             "ms_per_step": r["ms_per_step"], "steps": CONFIG_STEPS,
                             "warmup": CONFIG_WARMUP, "stage_ms": r["stage_ms"],
                             "expert_algorithm": "grouped gemm" if r["gemm"] else "weight streaming",
                             "roofline": g2, "roofline_down": d2, "layer_roofline": l2}
            print("config %s: %.1f us/step" % (name, r["ms_per_step"] * 1e3), file=sys.stderr,
                  flush=True)
            if name in FUSED_DECODE:
                fd = run_layer_fused_decode(c, CONFIG_STEPS, CONFIG_WARMUP, args.seed, moe, torch,
                                            dev)
                fd["step_time_ratio_to_separate_launches"] = (fd["ms_per_step"] /
                                                             r["ms_per_step"])
                configs[name]["fused_decode"] = fd
                print("config %s, fused decode: %.1f us/step" % (name, fd["ms_per_step"] * 1e3),
                      file=sys.stderr, flush=True)
            if name in BF16_COMPARISON:
                bf = run_layer_bf16(c, CONFIG_STEPS, CONFIG_WARMUP, args.seed, moe, torch, dev)
                bf["vs_mxfp4"] = bf16_comparison(c, configs[name], bf)
                configs["bf16_weights_" + name] = bf
                print("config %s, bf16 weights: %.1f us/step" % (name, bf["ms_per_step"] * 1e3),
                      file=sys.stderr, flush=True)
        result["configs"] = configs
        result["probes"] = probes(torch, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, run["inputs"])
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
