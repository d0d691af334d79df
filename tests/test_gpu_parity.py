"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: codes, scales, expert ids, histogram, offsets and permutations are
bit-exact (tokens whose oracle logits have a gap under 1e-4 among their
k+1 largest are excluded from id comparison, and the permutation is then
checked against the GPU's own ids); layer outputs satisfy
max|gpu - ref| <= 2^-7 (|ref| + rms(ref)) elementwise.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import mxfp4_quantized_mixture_amd as moe
from oracle import oracle as O
from synth import moe_inputs as MI
from tests import gpu_util as G
from tests import report

pytestmark = pytest.mark.gpu

FINITE = np.array([b for b in range(1 << 16) if ((b >> 7) & 0xFF) != 0xFF], np.uint16)
NEAR_TIE = 1e-4


def log(msg):
    print(msg, flush=True)


def gpu_quantize(w_bits, rule=0, stochastic=False, seed=0):
    q, s = moe.mxfp4_quantize(G.bf16_dev(w_bits), rule, stochastic=stochastic, seed=seed)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


# ------------------------------------------------------------------ quantize

@pytest.mark.parametrize("rule", [0, 1, 2])
def test_quantize_every_bf16_as_lone_element(rule):
    w = np.zeros((len(FINITE), 32), np.uint16)
    w[np.arange(len(FINITE)), np.arange(len(FINITE)) % 32] = FINITE
    q, s = gpu_quantize(w, rule)
    rq, rs = O.quantize(w, rule)
    assert np.array_equal(s, rs)
    assert np.array_equal(q, rq)


@pytest.mark.parametrize("rule", [0, 1, 2])
def test_quantize_every_bf16_under_many_maxima(rule):
    rows = []
    for E in (1, 2, 7, 60, 100, 118, 121, 124, 127, 130, 160, 200, 252, 253, 254):
        for M in (0, 63, 64, 127):
            mx = np.uint16(E << 7 | M)
            vals = FINITE[(FINITE & 0x7FFF) <= mx]
            n = (len(vals) + 30) // 31
            blk = np.zeros((n, 32), np.uint16)
            flat = np.zeros(n * 31, np.uint16)
            flat[:len(vals)] = vals
            blk[:, 1:] = flat.reshape(n, 31)
            blk[:, 0] = mx | (np.uint16(0x8000) if M == 63 else np.uint16(0))
            rows.append(blk)
    w = np.concatenate(rows)
    log("blocks: %d" % len(w))
    q, s = gpu_quantize(w, rule)
    rq, rs = O.quantize(w, rule)
    assert np.array_equal(s, rs)
    assert np.array_equal(q, rq)


@pytest.mark.parametrize("rule", [0, 1])
def test_quantize_random_rows_many_blocks(rule):
    rng = np.random.default_rng(21)
    v = rng.standard_normal((257, 2880)) * np.exp(rng.uniform(-40, 40, (257, 1)))
    w = MI.f32_to_bf16_bits(v.astype(np.float32))
    q, s = gpu_quantize(w, rule)
    rq, rs = O.quantize(w, rule)
    assert np.array_equal(s, rs) and np.array_equal(q, rq)


# Stochastic rounding: bit-exact against the oracle (same SplitMix64 stream,
# same threshold), over every finite bf16 value under many block maxima,
# random rows over 80 binades, the three scale rules and 64-bit seeds.
def _every_bf16_under_many_maxima():
    rows = []
    for E in (1, 2, 7, 60, 100, 118, 121, 124, 127, 130, 160, 200, 252, 253, 254):
        for M in (0, 63, 64, 65, 127):
            mx = np.uint16(E << 7 | M)
            vals = FINITE[(FINITE & 0x7FFF) <= mx]
            n = (len(vals) + 30) // 31
            blk = np.zeros((n, 32), np.uint16)
            flat = np.zeros(n * 31, np.uint16)
            flat[:len(vals)] = vals
            blk[:, 1:] = flat.reshape(n, 31)
            blk[:, 0] = mx | (np.uint16(0x8000) if M == 63 else np.uint16(0))
            rows.append(blk)
    return np.concatenate(rows)


@pytest.mark.parametrize("rule,seed", [(2, 0), (2, 0xFEDCBA9876543210), (0, 7), (1, 2 ** 63 + 5)])
def test_quantize_stochastic_every_bf16_under_many_maxima(rule, seed):
    w = _every_bf16_under_many_maxima()
    q, s = gpu_quantize(w, rule, stochastic=True, seed=seed)
    rq, rs = O.quantize(w, rule, stochastic=True, seed=seed)
    assert np.array_equal(s, rs)
    assert np.array_equal(q, rq)


@pytest.mark.parametrize("rule", [0, 1, 2])
def test_quantize_stochastic_random_rows(rule):
    rng = np.random.default_rng(23)
    v = rng.standard_normal((37, 2880)) * np.exp(rng.uniform(-40, 40, (37, 1)))
    w = MI.f32_to_bf16_bits(v.astype(np.float32))
    for seed in (1, 12345):
        q, s = gpu_quantize(w, rule, stochastic=True, seed=seed)
        rq, rs = O.quantize(w, rule, stochastic=True, seed=seed)
        assert np.array_equal(s, rs) and np.array_equal(q, rq), seed


def test_quantize_stochastic_seed_determines_the_codes():
    cfg = MI.CONFIGS["gptoss20b_decode"]
    w13, _ = MI.gen_expert(cfg, 0, 3)
    a = gpu_quantize(w13, 2, stochastic=True, seed=99)
    b = gpu_quantize(w13, 2, stochastic=True, seed=99)
    c = gpu_quantize(w13, 2, stochastic=True, seed=100)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[1], c[1]) and not np.array_equal(a[0], c[0])
    rq, rs = O.quantize(w13, 2, stochastic=True, seed=100)
    assert np.array_equal(c[0], rq) and np.array_equal(c[1], rs)


@pytest.mark.parametrize("name", ["tiny", "gptoss20b_decode", "gptoss120b_decode"])
def test_quantize_workload_experts(name):
    cfg = MI.CONFIGS[name]
    for e in (0, cfg.E - 1):
        w13, w2 = MI.gen_expert(cfg, 0, e)
        for w in (w13, w2):
            q, s = gpu_quantize(w)
            rq, rs = O.quantize(w)
            assert np.array_equal(s, rs) and np.array_equal(q, rq)
    if cfg.outliers:
        # outlier blocks raise their scale well above the N(0, 0.02) blocks
        assert rs.max() >= rs.min() + 4


def test_dequantize_matches_oracle():
    rng = np.random.default_rng(22)
    v = rng.standard_normal((64, 320)) * np.exp(rng.uniform(-20, 20, (64, 1)))
    w = MI.f32_to_bf16_bits(v.astype(np.float32))
    q, s = O.quantize(w)
    out = moe.mxfp4_dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda())
    got = G.bf16_bits_to_f64(G.bf16_host_bits(out))
    assert np.array_equal(got, O.dequantize(q, s))


def test_quantize_empty_and_errors():
    q, s = moe.mxfp4_quantize(torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda"))
    assert q.shape == (0, 32) and s.shape == (0, 2)
    with pytest.raises(moe.MoEError):
        moe.mxfp4_quantize(torch.zeros(4, 48, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(moe.MoEError):
        moe.mxfp4_quantize(torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda"), rule=3)


# ------------------------------------------------------------------ routing

def gpu_route(x, wr, b, k):
    r = moe.moe_route(G.bf16_dev(x), G.f32_dev(wr), None if b is None else G.f32_dev(b), k,
                      with_logits=True)
    torch.cuda.synchronize()
    return {f: getattr(r, f).cpu().numpy() for f in
            ("ids", "weights", "counts", "offsets", "sorted_pairs", "pair_pos", "logits")}


def check_route(x, wr, b, k, what):
    g = gpu_route(x, wr, b, k)
    ref = O.route(x, wr, b, k)
    T, E = ref["logits"].shape
    # logits: fp32 sum of D products against the fp64 one
    mag = G.bf16_bits_to_f64(x).__abs__() @ np.abs(wr.astype(np.float64)).T
    assert np.all(np.abs(g["logits"] - ref["logits"]) <= 3e-5 * mag + 1e-6), what
    near = ref["gap"] < NEAR_TIE
    ok = ~near
    assert np.array_equal(g["ids"][ok], ref["ids"][ok]), what
    # softmax over the selected logits: |dw_j| <= w_j (|dL_j| + sum_i w_i |dL_i|)
    # <= 2 w_j max_i |dL_i|, plus a few fp32 roundings of exp and the division
    dl = np.abs(np.take_along_axis(g["logits"] - ref["logits"], ref["ids"], 1)).max(1)
    wbound = 2.0 * ref["w"] * dl[:, None] + 8 * 2.0 ** -24 * ref["w"] + 2.0 ** -26
    assert np.all(np.abs(g["weights"][ok] - ref["w"][ok]) <= wbound[ok]), what
    # histogram / offsets / permutation against the GPU's own ids
    ids = g["ids"].ravel()
    cnt = np.bincount(ids, minlength=E)
    assert np.array_equal(g["counts"], cnt), what
    assert np.array_equal(g["offsets"], np.concatenate([[0], np.cumsum(cnt)])), what
    assert np.array_equal(g["sorted_pairs"], np.argsort(ids, kind="stable")), what
    assert np.array_equal(g["pair_pos"][g["sorted_pairs"]], np.arange(T * k)), what
    if not near.any():
        for a, b_ in (("counts", "counts"), ("offsets", "offsets"),
                      ("sorted_pairs", "sorted"), ("pair_pos", "pos")):
            assert np.array_equal(g[a], ref[b_]), (what, a)
    log("%s: T=%d E=%d k=%d near-tie tokens excluded: %d" % (what, T, E, k, int(near.sum())))
    return g, ref


ROUTE_CASES = ([("tiny", s) for s in range(10)] +
               [("gptoss20b_decode", s) for s in range(10)] +
               [("gptoss120b_decode", s) for s in range(10)] +
               [("gptoss20b_prefill", s) for s in range(3)] +
               [("gptoss120b_prefill_skewed", s) for s in range(3)])


@pytest.mark.parametrize("name,seed", ROUTE_CASES)
def test_route_workloads(name, seed):
    cfg = MI.CONFIGS[name]
    wr, b = MI.gen_router(cfg, seed)
    check_route(MI.gen_x(cfg, seed), wr, b, cfg.k, "%s/seed%d" % (name, seed))


# (T > 64 with D % 64 == 0 runs router_gemm_kernel: 32-expert blocks for E <= 32,
# 64-expert blocks otherwise, ragged in tokens and experts; other shapes the
# tile kernel)
@pytest.mark.parametrize("T,D,E,k", [(1, 32, 1, 1), (1, 64, 8, 8), (200, 96, 16, 3),
                                     (130, 64, 256, 8), (65, 32, 5, 5), (4096, 128, 64, 4),
                                     (333, 2880, 128, 4), (300, 128, 33, 2), (700, 4096, 40, 4)])
def test_route_shapes(T, D, E, k):
    rng = np.random.default_rng(T * 7 + E)
    x = MI.f32_to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    wr = (rng.standard_normal((E, D)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    check_route(x, wr, b, k, "shape T=%d D=%d E=%d k=%d" % (T, D, E, k))


@pytest.mark.parametrize("T", [70, 40])      # many-token path, and the one-block path (T <= 64)
def test_route_exact_ties_go_to_lower_id(T):
    D, E, k = 64, 12, 4
    x = np.zeros((T, D), np.uint16)
    wr = np.ones((E, D), np.float32)
    b = np.array([0.5, 2, 2, 1, 2, 0, 1, 1, 3, 0.5, 2, 3], np.float32)
    g = gpu_route(x, wr, b, k)
    assert np.array_equal(g["ids"], np.tile([8, 11, 1, 2], (T, 1)))
    ref = O.route(x, wr, b, k)
    for a, b_ in (("ids", "ids"), ("counts", "counts"), ("offsets", "offsets"),
                  ("sorted_pairs", "sorted"), ("pair_pos", "pos")):
        assert np.array_equal(g[a], ref[b_]), a


# The one-block routing kernel (T <= 64 and T*E <= 8192) is compiled once per
# k: every k, expert counts that leave wavefronts without experts (E < 16)
# or give them several, and both sides of its size limits.
SMALL_ROUTE = ([(64, 64, 2 * k + 3, k) for k in range(1, 9)] +
               [(17, 96, 128, 3), (32, 64, 256, 7), (64, 64, 128, 6),    # T*E = 8192
                (64, 64, 129, 5), (65, 64, 8, 2), (33, 2880, 200, 8)])


@pytest.mark.parametrize("T,D,E,k", SMALL_ROUTE)
def test_route_small_batches(T, D, E, k):
    rng = np.random.default_rng(1000 + T * 3 + E * 5 + k)
    x = MI.f32_to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    wr = (rng.standard_normal((E, D)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    check_route(x, wr, b, k, "small-batch T=%d D=%d E=%d k=%d" % (T, D, E, k))


# ------------------------------------------------------------------ full layer

class Inputs:
    def __init__(self, cfg, seed):
        self.cfg = cfg
        self.wr, self.b = MI.gen_router(cfg, seed)
        self.x = MI.gen_x(cfg, seed)
        self.w13, self.w2 = MI.gen_experts(cfg, seed, threads=G.THREADS)


def packed_ok(cfg):
    """Shapes whose expert weights the library takes in the packed layout."""
    return cfg.D % 64 == 0 and cfg.F % 64 == 0 and cfg.D <= 3840 and cfg.F <= 2944


def run_gpu_layer(inp, algo=moe.MLP_AUTO, packed=False):
    """Route and run the experts; returns the weights in row-major layout (for
    comparison with the oracle's codes) whichever layout the kernels read."""
    cfg = inp.cfg
    xd = G.bf16_dev(inp.x)
    weights = moe.ExpertWeights.quantize(G.bf16_dev(inp.w13), G.bf16_dev(inp.w2))
    r = moe.moe_route(xd, G.f32_dev(inp.wr), G.f32_dev(inp.b), cfg.k)
    out = moe.moe_expert_mlp(xd, weights.pack() if packed else weights, r, algo=algo)
    torch.cuda.synchronize()
    return weights, r, out


def tile_cover_tokens(r, k, every=16, small=8):
    """Tokens compared at full size: every `every`-th token, the tokens of the
    first and last sorted pair of every 128-pair tile of every expert (the
    grouped GEMM's tiles, from the GPU's own offsets), and every token of an
    expert with at most `small` pairs."""
    off = r.offsets.cpu().numpy()
    srt = r.sorted_pairs.cpu().numpy()
    T = r.ids.shape[0]
    toks = set(range(0, T, every))
    for e in range(len(off) - 1):
        beg, end = int(off[e]), int(off[e + 1])
        if end - beg <= small:
            toks |= set((srt[beg:end] // k).tolist())
        for t0 in range(beg, end, 128):
            toks.add(int(srt[t0]) // k)
            toks.add(int(srt[min(t0 + 128, end) - 1]) // k)
    return np.array(sorted(toks))


def assert_every_tile_compared(r, k, toks):
    """Every 128-pair tile of every expert has at least one compared row."""
    off = r.offsets.cpu().numpy()
    srt = r.sorted_pairs.cpu().numpy()
    cmp_ = np.zeros(r.ids.shape[0], bool)
    cmp_[toks] = True
    tiles = 0
    for e in range(len(off) - 1):
        for t0 in range(int(off[e]), int(off[e + 1]), 128):
            rows = srt[t0:min(t0 + 128, int(off[e + 1]))] // k
            assert cmp_[rows].any(), "expert %d tile at %d has no compared row" % (e, t0)
            tiles += 1
    return tiles


def reference_routing(inp, gids):
    """The oracle's routing, with the GPU's choice taken for tokens where the
    two differ.  That is allowed only where the choice is equally valid: every
    expert the GPU selected has an fp64 logit at least the largest unselected
    one minus twice the fp32 logit error bound (an fp32 dot product of length
    D: 3e-5 sum |x_d w_ed| + 1e-6).  Such tokens then use the softmax over the
    fp64 logits of the GPU's experts, in the GPU's slot order."""
    cfg = inp.cfg
    ref = O.route(inp.x, inp.wr, inp.b, cfg.k)
    ids = ref["ids"].copy()
    w = ref["w"].copy()
    L = ref["logits"]
    diff = np.nonzero((gids != ids).any(1))[0]
    if len(diff):
        mag = np.abs(G.bf16_bits_to_f64(inp.x[diff])) @ np.abs(inp.wr.astype(np.float64)).T
        bound = 3e-5 * mag.max(1) + 1e-6
        for i, t in enumerate(diff):
            sel = np.zeros(cfg.E, bool)
            sel[gids[t]] = True
            assert len(set(gids[t].tolist())) == cfg.k
            lo = L[t, sel].min()
            hi = L[t, ~sel].max() if (~sel).any() else -np.inf
            assert lo >= hi - 2 * bound[i], "token %d: GPU experts %s are not a valid top-%d" % (
                t, gids[t], cfg.k)
            ids[t] = gids[t]
            z = np.exp(L[t, gids[t]] - L[t, gids[t]].max())
            w[t] = z / z.sum()
    return ids, w, len(diff)


def check_layer(inp, tokens="all", what="", algo=moe.MLP_AUTO, packed=False):
    cfg = inp.cfg
    weights, r, out = run_gpu_layer(inp, algo, packed)
    gids = r.ids.cpu().numpy()
    ids, w, nswap = reference_routing(inp, gids)
    if tokens == "tiles":
        toks = tile_cover_tokens(r, cfg.k)
        ntiles = assert_every_tile_compared(r, cfg.k, toks)
    else:
        toks = np.arange(cfg.T)
        ntiles = None
    gq13, gs13 = weights.w13_q.cpu().numpy(), weights.w13_s.cpu().numpy()
    gq2, gs2 = weights.w2_q.cpu().numpy(), weights.w2_s.cpu().numpy()
    mismatched = []

    def expert_weights(e):
        q13, s13 = O.quantize(inp.w13[e])
        q2, s2 = O.quantize(inp.w2[e])
        if not (np.array_equal(q13, gq13[e]) and np.array_equal(s13, gs13[e]) and
                np.array_equal(q2, gq2[e]) and np.array_equal(s2, gs2[e])):
            mismatched.append(e)
        return q13, s13, q2, s2

    ref = O.moe_threaded(inp.x, expert_weights, ids, w, cfg.F, tokens=toks, threads=G.THREADS)
    assert not mismatched, "%s: quantized experts differ: %s" % (what, mismatched[:8])
    got = G.bf16_host_bits(out)[toks]
    worst = G.assert_within_tolerance(got, ref, what)
    msg = ("%s: %d of %d tokens compared%s, %d with the GPU's equally valid experts, "
           "max err/tol = %.3f" % (what, len(toks), cfg.T,
                                   "" if ntiles is None else " (covering all %d tiles)" % ntiles,
                                   nswap, worst))
    (report.note if cfg.D >= 2880 and cfg.T >= 32 else log)(msg)
    return out


@pytest.mark.parametrize("seed", range(10))
def test_layer_tiny(seed):
    check_layer(Inputs(MI.CONFIGS["tiny"], seed), what="tiny/seed%d" % seed)


# Full-size workloads in the layout the benchmark uses.  The prefill shapes
# compare every 16th token plus the first and last row of every 128-pair
# tile of every expert (so the tile table, the work remap across the XCDs
# and the 32-bit offsets are exercised at their real counts).
# Seeds: 0-9 for the decode shapes, 0-2 for the prefill shapes.
LAYER_CASES = ([("gptoss20b_decode", "all", s) for s in range(10)] +
               [("gptoss120b_decode", "all", s) for s in range(10)] +
               [("gptoss20b_prefill", "tiles", s) for s in range(3)] +
               [("gptoss120b_prefill_skewed", "tiles", s) for s in range(3)])


@pytest.mark.parametrize("name,tokens,seed", LAYER_CASES)
def test_layer_workloads(name, tokens, seed):
    # in the weight layout the benchmark uses: packed wherever the kernels take it
    cfg = MI.CONFIGS[name]
    check_layer(Inputs(cfg, seed), tokens=tokens, what="%s/seed%d" % (name, seed),
                packed=packed_ok(cfg))


EDGE = [
    MI.MoEConfig("ragged", T=37, D=96, F=160, E=6, k=2),
    MI.MoEConfig("one_expert_many_tokens", T=70, D=64, F=64, E=1, k=1),
    MI.MoEConfig("k_equals_E", T=20, D=128, F=96, E=4, k=4),
    MI.MoEConfig("single_token_full_width", T=1, D=2880, F=2880, E=32, k=4),
    MI.MoEConfig("wide_router", T=300, D=64, F=32, E=256, k=8),
    MI.MoEConfig("long_contraction_D", T=9, D=4096, F=64, E=2, k=1),
    MI.MoEConfig("long_contraction_F", T=9, D=64, F=4096, E=2, k=2),
    MI.MoEConfig("outliers_small", T=40, D=256, F=128, E=8, k=2, outliers=True),
    MI.MoEConfig("zipf_small", T=500, D=64, F=64, E=32, k=4, bias="zipf"),
]


@pytest.mark.parametrize("cfg", EDGE, ids=[c.name for c in EDGE])
def test_layer_edge_shapes(cfg):
    check_layer(Inputs(cfg, 3), what=cfg.name)


# Shapes for the grouped-GEMM path (128-pair tiles, 32-wide output fragments,
# 64-element contraction steps in groups of 3): ragged last tiles, tiles
# whose fragments leave wavefronts idle, step counts that are not multiples
# of 3, experts with a single pair, one expert with many tiles, E = 256.
GEMM_EDGE = [
    MI.MoEConfig("gemm_ragged", T=300, D=192, F=320, E=5, k=2),
    MI.MoEConfig("gemm_one_expert_many_tiles", T=1000, D=128, F=128, E=1, k=1),
    MI.MoEConfig("gemm_sparse_experts", T=40, D=64, F=64, E=64, k=2),
    MI.MoEConfig("gemm_skewed", T=2000, D=256, F=192, E=16, k=4, bias="zipf"),
    MI.MoEConfig("gemm_full_width", T=512, D=2880, F=2880, E=8, k=2),
    MI.MoEConfig("gemm_wide_router", T=700, D=128, F=64, E=256, k=8),
    MI.MoEConfig("gemm_outliers", T=256, D=512, F=256, E=4, k=2, outliers=True),
    MI.MoEConfig("gemm_long_contraction", T=300, D=4096, F=4160, E=2, k=1),
]


@pytest.mark.parametrize("cfg", GEMM_EDGE, ids=[c.name for c in GEMM_EDGE])
def test_layer_grouped_gemm_shapes(cfg):
    check_layer(Inputs(cfg, 4), what=cfg.name + "/grouped-gemm", algo=moe.MLP_GROUPED_GEMM)


def _random_shapes(n, seed):
    """Seeded random small layers that both expert algorithms take: D and F
    multiples of 64 (so every column range, wave and fragment count of the
    grouped GEMM occurs: D / 32 and F / 32 from 2 to 24), T from 1 to 700
    (short and many tiles), E up to 48, k up to min(E, 8); every fourth with
    the Zipf-like router bias (skewed expert loads)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 49))
        k = int(rng.integers(1, min(E, 8) + 1))
        out.append(MI.MoEConfig("random%d" % i, T=int(rng.integers(1, 701)),
                                D=64 * int(rng.integers(1, 13)), F=64 * int(rng.integers(1, 13)),
                                E=E, k=k, bias="zipf" if i % 4 == 3 else "zero"))
    return out


RANDOM_SHAPES = _random_shapes(32, 2024)


@pytest.mark.parametrize("cfg", RANDOM_SHAPES,
                         ids=["%s_T%d_D%d_F%d_E%d_k%d" % (c.name, c.T, c.D, c.F, c.E, c.k)
                              for c in RANDOM_SHAPES])
@pytest.mark.parametrize("algo", [moe.MLP_GROUPED_GEMM, moe.MLP_STREAM])
def test_layer_random_shapes(cfg, algo):
    check_layer(Inputs(cfg, 11), what="%s/algo %d" % (cfg.name, algo), algo=algo)


class W2ScaledInputs(Inputs):
    """Inputs whose W2 blocks are multiplied by powers of two (exact in
    bf16): "spread" draws a factor 2^(30 - r), r in [0, 40], per 32-element
    block, block 0 of every row taking 2^30 (so each row's blocks reach 40
    binades below its largest, and every row has the same top scale);
    "large" multiplies every W2 weight by 2^40, "small" by 2^-90.  The down
    contraction's block scales then leave fp16's range."""

    def __init__(self, cfg, seed, mode):
        super().__init__(cfg, seed)
        rng = np.random.default_rng(seed + 1000)
        w2 = MI.bf16_bits_to_f32(self.w2).reshape(cfg.E, cfg.D, cfg.F // 32, 32)
        if mode == "spread":
            r = 30.0 - rng.integers(0, 41, size=w2.shape[:3]).astype(np.float32)
            r[:, :, 0] = 30.0
        else:
            r = np.full(w2.shape[:3], 40.0 if mode == "large" else -90.0, np.float32)
        w2 = w2 * np.exp2(r)[..., None]
        self.w2 = MI.f32_to_bf16_bits(w2.reshape(cfg.E, cfg.D, cfg.F))


@pytest.mark.parametrize("mode", ["spread", "large", "small"])
@pytest.mark.parametrize("algo", [moe.MLP_GROUPED_GEMM, moe.MLP_STREAM])
def test_layer_w2_block_scales_outside_fp16_range(mode, algo):
    cfg = MI.MoEConfig("w2_scales", T=300, D=192, F=320, E=4, k=2)
    check_layer(W2ScaledInputs(cfg, 6, mode), what="w2 scales %s/algo %d" % (mode, algo),
                algo=algo)


class ScaledInputs(Inputs):
    """Inputs with W13 or x multiplied by powers of two (exact in bf16), so h
    and the outputs leave fp16's range (|h| about 2^40 or 2^-40 with W13
    x 2^+-20, 2^48 or 2^-48 with x x 2^+-24), or with every x element
    multiplied by its own 2^r, r uniform in [-16, 16], so the elements of a
    32-block span up to 32 binades."""

    def __init__(self, cfg, seed, mode):
        super().__init__(cfg, seed)
        rng = np.random.default_rng(seed + 2000)
        if mode.startswith("w13"):
            f = 2.0 ** float(mode[3:])
            self.w13 = MI.f32_to_bf16_bits(MI.bf16_bits_to_f32(self.w13) * np.float32(f))
        elif mode == "xwide":
            r = rng.integers(-16, 17, size=self.x.shape).astype(np.float32)
            self.x = MI.f32_to_bf16_bits(MI.bf16_bits_to_f32(self.x) * np.exp2(r))
        else:
            f = 2.0 ** float(mode[1:])
            self.x = MI.f32_to_bf16_bits(MI.bf16_bits_to_f32(self.x) * np.float32(f))


SCALE_MODES = ["w13+20", "w13-20", "x+24", "x-24", "xwide"]


@pytest.mark.parametrize("mode", SCALE_MODES)
@pytest.mark.parametrize("algo", [moe.MLP_GROUPED_GEMM, moe.MLP_STREAM])
def test_layer_activation_scales_outside_fp16_range(mode, algo):
    cfg = MI.MoEConfig("act_scales", T=300, D=192, F=320, E=4, k=2)
    check_layer(ScaledInputs(cfg, 7, mode), what="scaled %s/algo %d" % (mode, algo), algo=algo)


# A contraction longer than the streaming kernels take (F = 4160): the
# automatic choice runs the grouped GEMM, whatever the W2 block scales;
# naming the streaming algorithm is refused with MOE_ERR_SHAPE.
@pytest.mark.parametrize("w2_scale", [None, 30, -30, "spread"])
def test_layer_long_contraction_w2_scales(w2_scale):
    cfg = MI.MoEConfig("long_f", T=40, D=64, F=4160, E=2, k=1)
    if w2_scale == "spread":
        inp = W2ScaledInputs(cfg, 11, "spread")
    else:
        inp = Inputs(cfg, 11)
        if w2_scale is not None:
            inp.w2 = MI.f32_to_bf16_bits(MI.bf16_bits_to_f32(inp.w2) * np.float32(2.0 ** w2_scale))
    check_layer(inp, what="long_f w2 x 2^%s" % w2_scale)
    xd = G.bf16_dev(inp.x)
    w = moe.ExpertWeights.quantize(G.bf16_dev(inp.w13), G.bf16_dev(inp.w2))
    r = moe.moe_route(xd, G.f32_dev(inp.wr), G.f32_dev(inp.b), cfg.k)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_expert_mlp(xd, w, r, algo=moe.MLP_STREAM)
    assert ei.value.status == 2


@pytest.mark.parametrize("name", ["gemm_skewed", "gemm_full_width"])
def test_layer_streaming_on_gemm_shapes(name):
    cfg = {c.name: c for c in GEMM_EDGE}[name]
    check_layer(Inputs(cfg, 4), what=name + "/stream", algo=moe.MLP_STREAM)


@pytest.mark.parametrize("name", ["tiny", "gptoss20b_decode"])
def test_layer_grouped_gemm_on_decode_shapes(name):
    check_layer(Inputs(MI.CONFIGS[name], 2), what=name + "/grouped-gemm",
                algo=moe.MLP_GROUPED_GEMM)


def test_grouped_gemm_is_deterministic():
    inp = Inputs(GEMM_EDGE[3], 1)
    _, _, a = run_gpu_layer(inp, moe.MLP_GROUPED_GEMM)
    _, _, b = run_gpu_layer(inp, moe.MLP_GROUPED_GEMM)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# Contractions whose 64-wide step count leaves one or two stages after the
# grouped GEMM's three-stage loop (D/64 = 2 and 5, F/64 = 2 and 5), run
# repeatedly on workspaces pre-filled with NaN bytes or zeros: the h rows,
# y and the output must be the same every time (a stage that let its
# activation loads land after the barrier changed some h rows from run to
# run).
@pytest.mark.parametrize("D,F", [(128, 128), (320, 320), (128, 320)])
def test_grouped_gemm_tail_stages_repeatable(D, F):
    cfg = MI.MoEConfig("gemm_tail_%dx%d" % (D, F), T=1000, D=D, F=F, E=2, k=2)
    inp = Inputs(cfg, 9)
    xd = G.bf16_dev(inp.x)
    weights = moe.ExpertWeights.quantize(G.bf16_dev(inp.w13), G.bf16_dev(inp.w2))
    r = moe.moe_route(xd, G.f32_dev(inp.wr), G.f32_dev(inp.b), cfg.k)
    outs, wss = [], []
    for rep in range(6):
        ws = moe.mlp_workspace(cfg.T, D, F, cfg.E, cfg.k, xd.device)
        ws.fill_(0xFF if rep % 2 == 0 else 0)
        outs.append(moe.moe_expert_mlp(xd, weights, r, ws=ws, algo=moe.MLP_GROUPED_GEMM))
        wss.append(ws)
    torch.cuda.synchronize()
    P = cfg.T * cfg.k
    a256 = lambda v: (v + 255) // 256 * 256
    # what the grouped GEMM writes: y as fp16 [P, D], its scale bytes [P, D / 32],
    # then h as fp6 term rows (160 bytes per 64 elements, packed tile by tile)
    off_ys = a256(P * D * 2)
    off_h = a256(max(P * D * 4, off_ys + P * D // 32))
    regions = [(0, P * D * 2), (off_ys, off_ys + P * D // 32), (off_h, off_h + P * (F // 64) * 160)]
    for rep in range(1, 6):
        assert torch.equal(outs[rep].view(torch.int16), outs[0].view(torch.int16)), rep
        for a, b in regions:
            assert torch.equal(wss[rep][a:b], wss[0][a:b]), (rep, a, b)
    check_layer(inp, what=cfg.name + "/grouped-gemm", algo=moe.MLP_GROUPED_GEMM)


def test_layer_is_deterministic():
    inp = Inputs(MI.CONFIGS["gptoss20b_decode"], 1)
    _, _, a = run_gpu_layer(inp)
    _, _, b = run_gpu_layer(inp)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_moe_layer_object_matches_calls():
    inp = Inputs(MI.CONFIGS["tiny"], 2)
    cfg = inp.cfg
    weights, r, out = run_gpu_layer(inp)
    layer = moe.MoELayer(G.f32_dev(inp.wr), G.f32_dev(inp.b), weights, cfg.k, cfg.T)
    out2 = layer(G.bf16_dev(inp.x))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


# ------------------------------------------------------------ packed weights

def pack_reference(q):
    """mxfp4_pack's layout written with numpy: bytes [32t + 16h, 32t + 16h + 16)
    of row r of 32-row fragment f go to chunk (f, t), byte 512h + 16r of it."""
    rows, half = q.shape
    return np.ascontiguousarray(
        q.reshape(rows // 32, 32, half // 32, 2, 16).transpose(0, 2, 3, 1, 4)).reshape(rows, half)


@pytest.mark.parametrize("rows,K", [(32, 64), (96, 192), (64, 2880), (2 * 2880, 2880),
                                    (32 * 40, 4096)])
def test_pack_matches_reorder(rows, K):
    log("pack rows=%d K=%d" % (rows, K))
    q = np.random.default_rng(rows + K).integers(0, 256, (rows, K // 2), dtype=np.uint8)
    got = moe.mxfp4_pack(torch.from_numpy(q).cuda()).cpu().numpy()
    assert np.array_equal(got, pack_reference(q))


def test_pack_of_expert_stack_is_per_expert():
    # [E, R, K/2] packs as E*R rows; with R % 32 == 0 no fragment spans experts
    q = np.random.default_rng(1).integers(0, 256, (4, 96, 64), dtype=np.uint8)
    got = moe.mxfp4_pack(torch.from_numpy(q).cuda()).cpu().numpy()
    for e in range(4):
        assert np.array_equal(got[e], pack_reference(q[e]))


def test_pack_errors():
    with pytest.raises(moe.MoEError):
        moe.mxfp4_pack(torch.zeros(48, 32, dtype=torch.uint8, device="cuda"))    # rows % 32
    with pytest.raises(moe.MoEError):
        moe.mxfp4_pack(torch.zeros(32, 48, dtype=torch.uint8, device="cuda"))    # K % 64
    empty = moe.mxfp4_pack(torch.zeros(0, 32, dtype=torch.uint8, device="cuda"))
    assert empty.shape == (0, 32)


# The packed layout changes where the kernels load the codes, not what they
# compute: the layer output is bit-identical to the row-major run.
PACKED_CASES = [
    ("tiny", None), ("gptoss20b_decode", None), ("gemm_ragged", None),
    ("gemm_full_width", None), ("gemm_outliers", None),
    ("stream_max_lds", MI.MoEConfig("stream_max_lds", T=9, D=3840, F=2944, E=2, k=1)),
    ("sparse_experts", MI.MoEConfig("sparse_experts", T=5, D=128, F=192, E=64, k=3)),
]


@pytest.mark.parametrize("name,cfg", PACKED_CASES, ids=[c[0] for c in PACKED_CASES])
@pytest.mark.parametrize("algo", [moe.MLP_STREAM, moe.MLP_GROUPED_GEMM])
def test_packed_weights_bit_identical(name, cfg, algo):
    if cfg is None:
        cfg = MI.CONFIGS.get(name) or {c.name: c for c in GEMM_EDGE}[name]
    log("packed %s algo=%d" % (name, algo))
    inp = Inputs(cfg, 6)
    xd = G.bf16_dev(inp.x)
    w = moe.ExpertWeights.quantize(G.bf16_dev(inp.w13), G.bf16_dev(inp.w2))
    wp = w.pack()
    r = moe.moe_route(xd, G.f32_dev(inp.wr), G.f32_dev(inp.b), cfg.k)
    a = moe.moe_expert_mlp(xd, w, r, algo=algo)
    b = moe.moe_expert_mlp(xd, wp, r, algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(wp.w13_s, w.w13_s) and torch.equal(wp.w2_s, w.w2_s)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


def test_packed_weights_against_oracle_full_width_gemm():
    cfg = {c.name: c for c in GEMM_EDGE}["gemm_full_width"]
    check_layer(Inputs(cfg, 8), tokens="tiles", what="gemm_full_width/packed",
                algo=moe.MLP_GROUPED_GEMM, packed=True)


def test_packed_weights_rejected_where_the_kernels_cannot_take_them():
    cfg = MI.MoEConfig("too_wide", T=4, D=3904, F=64, E=2, k=1)
    inp = Inputs(cfg, 1)
    xd = G.bf16_dev(inp.x)
    w = moe.ExpertWeights.quantize(G.bf16_dev(inp.w13), G.bf16_dev(inp.w2)).pack()
    r = moe.moe_route(xd, G.f32_dev(inp.wr), G.f32_dev(inp.b), cfg.k)
    with pytest.raises(moe.MoEError):
        moe.moe_expert_mlp(xd, w, r)
