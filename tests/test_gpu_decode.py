"""GPU tests of the fused decode front (moe_layer_decode) through the C ABI.

Bar: bit-identical to moe_route followed by moe_expert_mlp with weight
streaming (MOE_MLP_STREAM) on the same inputs -- the output and every
routing array -- which the parity tests compare with the oracle; plus the
oracle directly on two workloads.  Also: many calls in a row on one
workspace (the control block resets itself), and a forced give-up of the
device-side waits (spin_limit = 0, set from the host) that must stay in
bounds, record the error, and leave the workspace usable after a re-init.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import mxfp4_quantized_mixture_amd as moe
from oracle import oracle as O
from synth import moe_inputs as MI
from tests import gpu_util as G
from tests.test_gpu_parity import Inputs, reference_routing

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


class Dev:
    """An Inputs set on the device, with MXFP4 weights (packed if asked)."""

    def __init__(self, inp, packed):
        self.inp, self.cfg = inp, inp.cfg
        self.x = G.bf16_dev(inp.x)
        self.wr, self.b = G.f32_dev(inp.wr), G.f32_dev(inp.b)
        w = moe.ExpertWeights.quantize(G.bf16_dev(inp.w13), G.bf16_dev(inp.w2))
        self.weights = w.pack() if packed else w


def two_launch(d):
    r = moe.moe_route(d.x, d.wr, d.b, d.cfg.k)
    out = moe.moe_expert_mlp(d.x, d.weights, r, algo=moe.MLP_STREAM)
    torch.cuda.synchronize()
    return out, r


def fused(d, ws=None, spin_limit=moe.DECODE_SPIN_LIMIT):
    out, r = moe.moe_layer_decode(d.x, d.wr, d.b, d.weights, d.cfg.k, ws=ws,
                                  spin_limit=spin_limit)
    torch.cuda.synchronize()
    return out, r


def same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def assert_identical(d, got, want, what):
    (o1, r1), (o2, r2) = got, want
    for name in ("ids", "weights", "counts", "offsets", "sorted_pairs", "pair_pos"):
        assert same(getattr(r1, name), getattr(r2, name)), "%s: %s differ" % (what, name)
    assert same(o1, o2), "%s: outputs differ" % what


def packed_ok(cfg):
    return cfg.D % 64 == 0 and cfg.F % 64 == 0 and cfg.D <= 3840 and cfg.F <= 2944


DECODE_SHAPES = [
    MI.CONFIGS["tiny"],
    MI.CONFIGS["gptoss20b_decode"],
    MI.CONFIGS["gptoss120b_decode"],
    MI.MoEConfig("one_token", T=1, D=2880, F=2880, E=32, k=4),
    MI.MoEConfig("ragged", T=37, D=96, F=160, E=6, k=2),
    MI.MoEConfig("wide_router_k8", T=32, D=64, F=32, E=256, k=8),
    MI.MoEConfig("crowded_expert", T=64, D=128, F=128, E=2, k=1),
    MI.MoEConfig("max_tokens_120b", T=64, D=2880, F=2880, E=128, k=4),
]


@pytest.mark.parametrize("cfg", DECODE_SHAPES, ids=[c.name for c in DECODE_SHAPES])
def test_decode_bit_identical_to_two_launches(cfg):
    d = Dev(Inputs(cfg, 6), packed=packed_ok(cfg))
    ws = moe.decode_workspace(cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, G.device())
    got = fused(d, ws)
    assert moe.decode_error(ws) == 0
    assert_identical(d, got, two_launch(d), cfg.name)
    log("%s: fused decode bit-identical (packed=%s)" % (cfg.name, packed_ok(cfg)))


def test_decode_canonical_codes_bit_identical():
    cfg = MI.CONFIGS["gptoss20b_decode"]
    d = Dev(Inputs(cfg, 7), packed=False)
    assert_identical(d, fused(d), two_launch(d), "canonical codes")


@pytest.mark.parametrize("name", ["tiny", "gptoss20b_decode"])
def test_decode_against_oracle(name):
    cfg = MI.CONFIGS[name]
    inp = Inputs(cfg, 8)
    d = Dev(inp, packed=packed_ok(cfg))
    out, r = fused(d)
    ids, w, nswap = reference_routing(inp, r.ids.cpu().numpy())

    def expert_weights(e):
        q13, s13 = O.quantize(inp.w13[e])
        q2, s2 = O.quantize(inp.w2[e])
        return q13, s13, q2, s2

    ref = O.moe_threaded(inp.x, expert_weights, ids, w, cfg.F, threads=G.THREADS)
    worst = G.assert_within_tolerance(G.bf16_host_bits(out), ref, name)
    log("%s: fused decode vs oracle, max err/tol = %.3f (%d swapped)" % (name, worst, nswap))


def test_decode_many_calls_on_one_workspace():
    cfg = MI.CONFIGS["gptoss20b_decode"]
    a = Dev(Inputs(cfg, 9), packed=True)
    b = Dev(Inputs(cfg, 10), packed=True)
    ws = moe.decode_workspace(cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, G.device())
    want = {id(a): two_launch(a), id(b): two_launch(b)}
    for i in range(12):
        d = a if i % 3 else b
        assert_identical(d, fused(d, ws), want[id(d)], "call %d" % i)
    assert moe.decode_error(ws) == 0
    ctl = ws[:16].view(torch.int32).cpu().numpy()
    assert np.all(ctl == 0), "control block not reset: %s" % ctl


def test_decode_forced_give_up_stays_in_bounds_and_recovers():
    cfg = MI.CONFIGS["gptoss20b_decode"]
    d = Dev(Inputs(cfg, 11), packed=True)
    ws = moe.decode_workspace(cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, G.device())
    want = two_launch(d)
    gave_up = 0
    for _ in range(3):
        out, r = fused(d, ws, spin_limit=0)        # every wait looks once
        err = moe.decode_error(ws)
        if err == 0:
            assert_identical(d, (out, r), want, "spin_limit=0 without a give-up")
        else:
            gave_up += 1
            off = r.offsets.cpu().numpy()
            assert off.min() >= 0 and off.max() <= cfg.T * cfg.k
        moe.decode_init(ws)
    log("spin_limit = 0: %d of 3 calls gave up" % gave_up)
    assert_identical(d, fused(d, ws), want, "after re-init")
    assert moe.decode_error(ws) == 0
