"""GPU parity of the bf16-weight comparison path (moe_expert_mlp_bf16)
against the oracle's bf16-weight experts, through the C ABI.

Bar: x and the weights enter exactly and every product is exact, so apart
from fp32 accumulation (and h's two-term bf16 split, below 2^-17 of |h|) the
only rounding is the output's bf16 rounding, at most 2^-8 of |out| (bf16's
unit roundoff: 8 significant bits):
max|gpu - ref| <= 2^-8 |ref| + 2^-11 rms(ref) elementwise.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import mxfp4_quantized_mixture_amd as moe
from oracle import oracle as O
from synth import moe_inputs as MI
from tests import gpu_util as G
from tests.test_gpu_parity import Inputs, reference_routing, tile_cover_tokens

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def run_gpu_bf16(inp):
    cfg = inp.cfg
    xd = G.bf16_dev(inp.x)
    r = moe.moe_route(xd, G.f32_dev(inp.wr), G.f32_dev(inp.b), cfg.k)
    out = moe.moe_expert_mlp_bf16(xd, G.bf16_dev(inp.w13), G.bf16_dev(inp.w2), r)
    torch.cuda.synchronize()
    return r, out


def check_bf16(inp, what, tokens="all"):
    cfg = inp.cfg
    r, out = run_gpu_bf16(inp)
    ids, w, nswap = reference_routing(inp, r.ids.cpu().numpy())
    toks = tile_cover_tokens(r, cfg.k) if tokens == "tiles" else np.arange(cfg.T)
    ref = O.moe_threaded(inp.x, lambda e: (inp.w13[e], inp.w2[e]), ids, w, cfg.F, tokens=toks,
                         threads=G.THREADS)
    got = G.bf16_bits_to_f64(G.bf16_host_bits(out)[toks])
    assert np.all(np.isfinite(got)), what
    rms = float(np.sqrt(np.mean(ref * ref)))
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -11 * rms
    ratio = np.abs(got - ref) / tol
    worst = float(ratio.max())
    log("%s: %d of %d tokens, %d with the GPU's equally valid experts, max err/tol = %.3f"
        % (what, len(toks), cfg.T, nswap, worst))
    assert worst <= 1.0, "%s: max err/tol = %.3f at %s" % (
        what, worst, np.unravel_index(int(ratio.argmax()), ratio.shape))
    return out


@pytest.mark.parametrize("seed", range(3))
def test_bf16_layer_tiny(seed):
    check_bf16(Inputs(MI.CONFIGS["tiny"], seed), "tiny/seed%d" % seed)


@pytest.mark.parametrize("name", ["gptoss20b_decode", "gptoss120b_decode"])
def test_bf16_layer_decode_workloads(name):
    check_bf16(Inputs(MI.CONFIGS[name], 0), name)


# Work split: 16-row tiles over 8 wavefronts per block, experts in groups of
# 16 pairs (several groups per expert, one pair, none), contraction steps of
# 32 with batches of 4 and ragged tails, long contractions, E = 256, k = 8.
BF16_EDGE = [
    MI.MoEConfig("ragged", T=37, D=96, F=160, E=6, k=2),
    MI.MoEConfig("one_expert_many_groups", T=70, D=64, F=64, E=1, k=1),
    MI.MoEConfig("k_equals_E", T=20, D=128, F=96, E=4, k=4),
    MI.MoEConfig("single_token_full_width", T=1, D=2880, F=2880, E=32, k=4),
    MI.MoEConfig("wide_router", T=300, D=64, F=32, E=256, k=8),
    MI.MoEConfig("long_contraction_D", T=9, D=4096, F=64, E=2, k=1),
    MI.MoEConfig("long_contraction_F", T=9, D=64, F=4160, E=2, k=2),
    MI.MoEConfig("outliers_small", T=40, D=256, F=128, E=8, k=2, outliers=True),
    MI.MoEConfig("zipf_small", T=500, D=64, F=64, E=32, k=4, bias="zipf"),
    MI.MoEConfig("many_groups", T=512, D=256, F=288, E=4, k=2),
]


@pytest.mark.parametrize("cfg", BF16_EDGE, ids=[c.name for c in BF16_EDGE])
def test_bf16_layer_edge_shapes(cfg):
    check_bf16(Inputs(cfg, 5), cfg.name)


def test_bf16_layer_is_deterministic():
    inp = Inputs(MI.CONFIGS["gptoss20b_decode"], 1)
    _, a = run_gpu_bf16(inp)
    _, b = run_gpu_bf16(inp)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_bf16_prepared_layer_matches_calls():
    cfg = MI.CONFIGS["gptoss20b_decode"]
    inp = Inputs(cfg, 2)
    xd = G.bf16_dev(inp.x)
    wr, b = G.f32_dev(inp.wr), G.f32_dev(inp.b)
    w13, w2 = G.bf16_dev(inp.w13), G.bf16_dev(inp.w2)
    r0, want = run_gpu_bf16(inp)
    out = torch.empty(cfg.T, cfg.D, dtype=torch.bfloat16, device=G.device())
    routing = moe.alloc_routing(cfg.T, cfg.E, cfg.k, G.device())
    layer = moe.PreparedLayer(xd, wr, b, (w13, w2), cfg.k, out, routing,
                              moe.route_workspace(cfg.T, cfg.D, cfg.E, cfg.k, G.device()),
                              moe.mlp_bf16_workspace(cfg.T, cfg.D, cfg.F, cfg.E, cfg.k,
                                                     G.device()))
    layer()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
