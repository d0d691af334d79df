"""Throughput of the MXFP4 MoE layer (route + experts + combine) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole layer -- moe_route then moe_expert_mlp --
over one batch of synthetic tokens already resident in HBM.  The default
workload is the GPT-OSS-20B-shaped decode step (T=32 tokens, d_model = d_ff =
2880, 32 experts, top-4).  Expert weights are quantized to MXFP4 once,
outside the timed region, and NCOPIES copies are rotated step to step so the
256 MB last-level cache cannot hold the weights between steps.

Prints one JSON line.  `value` is tokens/s of the whole layer; `roofline`
prices the dominant kernel (the gate/up expert kernel) using algorithmic
bytes / flops and the kernel's own duration from HIP events recorded on its
stream in the timed region: against HBM bandwidth when the layer streams
the expert weights (few pairs per expert), against the matrix cores' fp8
rate when it runs the grouped GEMM (the block-scaled fp4 x fp8 products
issue at the fp8 rate).  `cpu_baseline` is the single-threaded CPU oracle on
the same workload (the whole decode step, or a token sample for prefill
workloads).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 matrix cores, TFLOP/s
NCOPIES = 3


def algorithmic_work(cfg, counts: np.ndarray) -> dict:
    """Bytes the layer must move and flops it must do (intermediates excluded)."""
    D, F, E, T, k = cfg.D, cfg.F, cfg.E, cfg.T, cfg.k
    touched = int((counts > 0).sum())
    w13_bytes = 2 * F * (D // 2 + D // 32)     # codes + E8M0 scales of one expert
    w2_bytes = D * (F // 2 + F // 32)
    x_bytes = 2 * T * D
    step_bytes = touched * (w13_bytes + w2_bytes) + 4 * E * D + 4 * E + x_bytes + 2 * T * D
    gateup_bytes = touched * w13_bytes + x_bytes
    pairs = T * k
    return dict(touched=touched, step_bytes=step_bytes, gateup_bytes=gateup_bytes,
                step_flops=6 * D * F * pairs, gateup_flops=4 * D * F * pairs)


def packed_ok(cfg) -> bool:
    """Shapes the library accepts with packed weight codes (both expert
    algorithms: contraction sizes multiples of 64 within the streaming
    kernels' LDS budget)."""
    return cfg.D % 64 == 0 and cfg.F % 64 == 0 and cfg.D <= 3840 and cfg.F <= 2944


def read_traffic(kernel: str, workload: str, source: str, layout: str):
    """HBM bytes per dispatch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source with the same weight layout (else
    None)."""
    path = os.path.join(ROOT, "profiles", "%s.%s.traffic.txt" % (kernel, workload))
    src = os.path.join(ROOT, "mxfp4_quantized_mixture_amd", "csrc", source)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != digest or fields.get("weight_layout") != layout:
        return None
    try:
        return float(fields["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, inp, tokens) -> dict:
    """The CPU oracle as it is (single-threaded C, fp64) on the same inputs."""
    from oracle import oracle as orc
    from concurrent.futures import ThreadPoolExecutor

    x, wr, b, w13, w2 = inp
    # oracle-side quantization is input preparation, not timed
    with ThreadPoolExecutor(max_workers=16) as ex:
        q13 = list(ex.map(lambda e: orc.quantize(w13[e]), range(cfg.E)))
        q2 = list(ex.map(lambda e: orc.quantize(w2[e]), range(cfg.E)))
    q13q = np.stack([a for a, _ in q13]); q13s = np.stack([s for _, s in q13])
    q2q = np.stack([a for a, _ in q2]); q2s = np.stack([s for _, s in q2])
    t0 = time.perf_counter()
    r = orc.route(x, wr, b, cfg.k)
    orc.moe(x, q13q, q13s, q2q, q2s, r["ids"], r["w"], cfg.F,
            tokens=None if tokens is None else np.asarray(tokens, np.int32))
    dt = time.perf_counter() - t0
    n = cfg.T if tokens is None else len(tokens)
    what = ("whole step: %d tokens routed (router over all %d tokens), %d expert pairs, "
            "combine" % (n, cfg.T, n * cfg.k))
    return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": what, "seconds": dt, "host_cpu": platform.processor() or platform.machine()}


def bench_quantize(cfg, args, moe, torch, dev) -> int:
    """mxfp4_quantize of all the workload's expert weights, W13 [E*2F, D] and
    W2 [E*D, F] bf16 (one call each per step), both roundings; HBM bytes =
    2 B read per element + 0.5 + 1/32 B written."""
    from synth import moe_inputs as MI
    w13, w2 = MI.gen_experts(cfg, args.seed, threads=16)
    mats = [torch.from_numpy(a.reshape(-1, a.shape[-1]).view(np.int16)).to(dev).view(torch.bfloat16)
            for a in (w13, w2)]
    del w13, w2
    elems = sum(m.numel() for m in mats)
    nbytes = elems * 2 + elems // 2 + elems // 32
    out = {}
    for name, kw in (("nearest_even", {}), ("stochastic", {"stochastic": True, "seed": 1})):
        rule = moe.SCALE_CEIL_DIV6 if kw else moe.SCALE_FLOOR_DIV6
        for _ in range(max(args.warmup // 10, 2)):
            for m in mats:
                moe.mxfp4_quantize(m, rule, **kw)
        n = max(args.steps // 20, 5)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(n):
            for m in mats:
                moe.mxfp4_quantize(m, rule, **kw)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / n
        out[name] = {"ms": ms, "GB/s": nbytes / (ms * 1e-3) / 1e9,
                     "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    print(json.dumps({"metric": "mxfp4_quantize HBM GB/s",
                      "workload": "%s: all %d experts' W13 and W2" % (cfg.name, cfg.E),
                      "matrices": [list(m.shape) for m in mats], "bytes_per_step": nbytes,
                      "steps": n, "results": out}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gptoss20b_decode")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--algo", default="auto", choices=["auto", "stream", "gemm"],
                    help="expert algorithm (default: the library's automatic choice)")
    ap.add_argument("--layout", default="auto", choices=["auto", "canonical", "packed"],
                    help="expert weight code layout (default: packed where the kernels take it)")
    ap.add_argument("--quantize", action="store_true",
                    help="time mxfp4_quantize (nearest-even and stochastic rounding) on the "
                         "workload's expert weights (W13 and W2) instead of the layer")
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
    cfg = MI.CONFIGS[args.workload]
    if args.quantize:
        return bench_quantize(cfg, args, moe, torch, dev)
    wr, b = MI.gen_router(cfg, args.seed)
    x = MI.gen_x(cfg, args.seed)
    w13, w2 = MI.gen_experts(cfg, args.seed, threads=16)

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    xd, wrd, bd = bf16(x), torch.from_numpy(wr).to(dev), torch.from_numpy(b).to(dev)
    packed = args.layout == "packed" or (args.layout == "auto" and packed_ok(cfg))
    layout = "packed" if packed else "row-major"
    base = moe.ExpertWeights.quantize(bf16(w13), bf16(w2), packed=packed)
    copies = [base] + [moe.ExpertWeights(base.w13_q.clone(), base.w13_s.clone(),
                                         base.w2_q.clone(), base.w2_s.clone(), packed)
                       for _ in range(NCOPIES - 1)]
    out = torch.empty(cfg.T, cfg.D, dtype=torch.bfloat16, device=dev)
    routing = moe.alloc_routing(cfg.T, cfg.E, cfg.k, dev)
    route_ws = moe.route_workspace(cfg.T, cfg.D, cfg.E, cfg.k, dev)
    mlp_ws = moe.mlp_workspace(cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, dev)
    algo = {"auto": moe.MLP_AUTO, "stream": moe.MLP_STREAM,
            "gemm": moe.MLP_GROUPED_GEMM}[args.algo]
    layers = [moe.PreparedLayer(xd, wrd, bd, w, cfg.k, out, routing, route_ws, mlp_ws, algo=algo)
              for w in copies]
    torch.cuda.synchronize()

    for i in range(args.warmup):
        layers[i % NCOPIES]()
    K = args.steps
    # Timed region 1 (value): the layer alone, nothing else on the stream.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        layers[i % NCOPIES]()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    # Timed region 2 (per-kernel durations): the same K steps with HIP events
    # recorded on the layer's stream around each expert kernel.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    evarr = [moe.PreparedLayer.event_array(e) for e in ev]
    torch.cuda.synchronize()
    for i in range(K):
        layers[i % NCOPIES](evarr[i])
    torch.cuda.synchronize()
    gateup_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    down_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    combine_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    ms_per_step = total_ms / K

    counts = routing.counts.cpu().numpy()
    work = algorithmic_work(cfg, counts)
    # the library's automatic choice: the grouped GEMM once the average expert
    # receives 32 pairs, weight streaming below that
    decode = (args.algo == "stream" or
              (args.algo == "auto" and cfg.T * cfg.k < 32 * cfg.E))
    if decode:
        ach = work["gateup_bytes"] / (gateup_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS}
        layer = work["step_bytes"] / (ms_per_step * 1e-3) / 1e9
        layer_roof = {"bound": "hbm", "achieved": layer, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": layer / HBM_PEAK_GBS}
    else:
        ach = work["gateup_flops"] / (gateup_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / FP8_PEAK_TFLOPS,
                # x enters as 2 exact fp8 terms: the matrix cores execute twice the flops
                "executed_tflops": 2 * ach}
        layer = work["step_flops"] / (ms_per_step * 1e-3) / 1e12
        layer_roof = {"bound": "mfma", "achieved": layer, "peak": FP8_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": layer / FP8_PEAK_TFLOPS}
    if decode:
        roof["kernel"] = "expert_stream_kernel<gate_up%s>" % (",packed" if packed else "")
        roof["traffic"] = read_traffic("gateup", cfg.name, "expert_mlp.hip", layout)
    else:
        roof["kernel"] = "expert_gemm_kernel<gate_up%s>" % (",packed" if packed else "")
        roof["traffic"] = read_traffic("gateup_gemm", cfg.name, "expert_gemm.hip", layout)
    roof["algorithmic_per_launch"] = work["gateup_bytes"] if decode else work["gateup_flops"]
    roof["avg_launch_ms"] = gateup_ms

    result = {
        "metric": "MXFP4 MoE-layer tokens/s",
        "value": cfg.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4*fp8->f32" if decode else "mxfp4*fp8->f32 (gate/up), f16*f16->f32 (down)",
        "data": "synthetic",
        "config": {"workload": cfg.description, "name": cfg.name, "tokens": cfg.T,
                   "d_model": cfg.D, "d_ff": cfg.F, "experts": cfg.E, "top_k": cfg.k,
                   "expert_weights": "mxfp4 (e2m1 + e8m0 per 32)",
                   "matrix_cores": ("block-scaled mfma: mxfp4 weights x fp8 residual terms "
                                    "of the activations, fp32 accumulate") if decode else
                                   ("gate/up: block-scaled mfma, mxfp4 weights x 2 fp8 terms "
                                    "of x; down: f16 mfma, fp16 h x W2 codes converted to "
                                    "fp16 per tile; fp32 accumulate"),
                   "expert_algorithm": "weight streaming" if decode else "grouped gemm",
                   "weight_layout": "packed 32x64 fragments" if packed else "row-major",
                   "touched_experts": work["touched"], "weight_copies_rotated": NCOPIES,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer_roofline": layer_roof,
        "stage_ms": {"gate_up": gateup_ms, "down": down_ms, "combine": combine_ms},
    }
    if not args.no_cpu_baseline:
        tokens = None
        if cfg.T > 64:
            rng = np.random.default_rng(0)
            tokens = np.sort(rng.choice(cfg.T, size=16, replace=False))
        result["cpu_baseline"] = cpu_baseline(cfg, (x, wr, b, w13, w2), tokens)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
