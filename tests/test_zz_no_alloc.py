"""moe_expert_mlp_noalloc: the same results as moe_expert_mlp_ex with a
caller-owned workspace, on two calls in a row (the second smaller, so it
runs on whatever the first left in the fixed workspace), for both expert
algorithms and both weight layouts; and a size beyond the fixed workspace is
refused before anything is enqueued."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import mxfp4_quantized_mixture_amd as moe
from synth import moe_inputs as MI
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _layer(cfg, seed):
    wr, b = MI.gen_router(cfg, seed)
    x = MI.gen_x(cfg, seed)
    w13, w2 = MI.gen_experts(cfg, seed, threads=G.THREADS)
    xd = G.bf16_dev(x)
    w = moe.ExpertWeights.quantize(G.bf16_dev(w13), G.bf16_dev(w2))
    r = moe.moe_route(xd, G.f32_dev(wr), G.f32_dev(b), cfg.k)
    return xd, w, r


CASES = [
    # (first call, second call): the second is smaller
    (MI.MoEConfig("na_decode", T=64, D=2880, F=2880, E=32, k=4),
     MI.MoEConfig("na_decode_small", T=5, D=2880, F=2880, E=32, k=4)),
    (MI.MoEConfig("na_gemm", T=600, D=256, F=192, E=4, k=2),
     MI.MoEConfig("na_gemm_small", T=150, D=256, F=192, E=4, k=2)),
]


@pytest.mark.parametrize("algo", [moe.MLP_AUTO, moe.MLP_STREAM, moe.MLP_GROUPED_GEMM])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("big,small", CASES, ids=[c[0].name for c in CASES])
def test_noalloc_matches_workspace_call_twice(big, small, algo, packed):
    outs = []
    for i, cfg in enumerate((big, small)):
        xd, w, r = _layer(cfg, 3 + i)
        if packed:
            w = w.pack()
        ref = moe.moe_expert_mlp(xd, w, r, algo=algo)
        ws_need = moe.lib().moe_expert_mlp_workspace_size(cfg.T, cfg.D, cfg.F, cfg.E, cfg.k)
        assert ws_need <= moe.NOALLOC_SCRATCH_BYTES
        out = torch.full_like(ref, float("nan"))
        moe.moe_expert_mlp_noalloc(xd, w, r, out, algo=algo)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (cfg.name, algo, packed)
        outs.append(out)
    assert all(torch.isfinite(o.float()).all() for o in outs)


def test_noalloc_refuses_sizes_beyond_its_workspace():
    cfg = MI.MoEConfig("na_too_big", T=169, D=2880, F=2880, E=32, k=4)
    assert moe.lib().moe_expert_mlp_workspace_size(cfg.T, cfg.D, cfg.F, cfg.E, cfg.k) > \
        moe.NOALLOC_SCRATCH_BYTES
    dev = G.device()
    x = torch.zeros(cfg.T, cfg.D, dtype=torch.bfloat16, device=dev)
    w = moe.ExpertWeights(torch.zeros(cfg.E, 2 * cfg.F, cfg.D // 2, dtype=torch.uint8, device=dev),
                          torch.zeros(cfg.E, 2 * cfg.F, cfg.D // 32, dtype=torch.uint8, device=dev),
                          torch.zeros(cfg.E, cfg.D, cfg.F // 2, dtype=torch.uint8, device=dev),
                          torch.zeros(cfg.E, cfg.D, cfg.F // 32, dtype=torch.uint8, device=dev))
    r = moe.alloc_routing(cfg.T, cfg.E, cfg.k, dev)
    out = torch.zeros(cfg.T, cfg.D, dtype=torch.bfloat16, device=dev)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_expert_mlp_noalloc(x, w, r, out)
    assert ei.value.status == 3
    torch.cuda.synchronize()
    assert not out.view(torch.int16).any()              # nothing was enqueued
