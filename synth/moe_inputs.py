"""Seeded synthetic inputs for the MXFP4 mixture-of-experts MLP layer.

This module only draws random numbers and rounds them to the storage types
the layer takes as input (fp32 router weights, bf16 activations, bf16 expert
weights before quantization).  It holds none of the layer's arithmetic, so
both the CPU oracle and the GPU path can be fed from it.

Recipe (one generator per stream, NumPy PCG64 seeded with
``SeedSequence([seed, stream, ...])``):

* stream 0 -- router weight Wr[E, D]: N(0, 0.02^2) drawn in fp64, rounded to
  fp32.
* router bias b[E]: zero, or for the skewed-routing workload the Zipf-like
  b_e = 1.5 * ln(1 / (e + 1)^1.2) computed in fp64 and rounded to fp32.
* stream 2 / 3 -- expert e's W13[2F, D] (gate rows, then up rows) and
  W2[D, F]: standard normals drawn in fp32 (``standard_normal(dtype=float32)``)
  times float32(0.02), then rounded to bf16 (round half to even).  Each
  expert has its own sub-stream ``[seed, stream, e]`` so one expert can be
  regenerated alone.
* stream 5 -- outliers (120B-shaped decode workload only): in each expert's
  W13 and W2, 1 % of the 32-element blocks along the contraction dimension
  (chosen without replacement) get one uniformly chosen element multiplied by
  50 before the bf16 rounding.
* stream 4 -- activations x[T, D]: N(0, 1) drawn in fp32, rounded to bf16.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int          # tokens
    D: int          # d_model
    F: int          # d_ff (per expert)
    E: int          # experts
    k: int          # experts per token
    bias: str = "zero"        # "zero" | "zipf"
    outliers: bool = False    # x50 outlier element in 1 % of blocks
    description: str = ""

    @property
    def P(self) -> int:
        return self.T * self.k


CONFIGS = {
    "tiny": MoEConfig(
        "tiny", T=16, D=64, F=64, E=8, k=2,
        description="tiny MoE layer, T=16 D=F=64 E=8 top-2"),
    "gptoss20b_decode": MoEConfig(
        "gptoss20b_decode", T=32, D=2880, F=2880, E=32, k=4,
        description="GPT-OSS-20B-shaped MoE decode step, T=32 D=F=2880 E=32 top-4"),
    "gptoss120b_decode": MoEConfig(
        "gptoss120b_decode", T=64, D=2880, F=2880, E=128, k=4, outliers=True,
        description="GPT-OSS-120B-shaped MoE decode, T=64 D=F=2880 E=128 top-4, "
                    "x50 outliers in 1% of weight blocks"),
    "gptoss20b_prefill": MoEConfig(
        "gptoss20b_prefill", T=8192, D=2880, F=2880, E=32, k=4,
        description="GPT-OSS-20B-shaped prefill, T=8192 D=F=2880 E=32 top-4"),
    "gptoss120b_prefill_skewed": MoEConfig(
        "gptoss120b_prefill_skewed", T=16384, D=2880, F=2880, E=128, k=4, bias="zipf",
        description="GPT-OSS-120B-shaped prefill with Zipf-biased routing, "
                    "T=16384 D=F=2880 E=128 top-4"),
}

STREAM_ROUTER, STREAM_W13, STREAM_W2, STREAM_X, STREAM_OUTLIER = 0, 2, 3, 4, 5


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (round half to even); return bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gen_router(cfg: MoEConfig, seed: int) -> tuple[np.ndarray, np.ndarray]:
    wr = (_rng(seed, STREAM_ROUTER).standard_normal((cfg.E, cfg.D)) * 0.02).astype(np.float32)
    if cfg.bias == "zipf":
        e = np.arange(cfg.E, dtype=np.float64)
        b = (1.5 * np.log(1.0 / (e + 1.0) ** 1.2)).astype(np.float32)
    else:
        b = np.zeros(cfg.E, dtype=np.float32)
    return wr, b


def gen_x(cfg: MoEConfig, seed: int) -> np.ndarray:
    x = _rng(seed, STREAM_X).standard_normal((cfg.T, cfg.D), dtype=np.float32)
    return f32_to_bf16_bits(x)


def _plant_outliers(w: np.ndarray, rng: np.random.Generator) -> None:
    """Multiply one element in 1 % of the 32-blocks of w [rows, K] by 50."""
    rows, K = w.shape
    nblk = rows * (K // 32)
    m = int(round(0.01 * nblk))
    blocks = rng.choice(nblk, size=m, replace=False)
    lane = rng.integers(0, 32, size=m)
    flat = w.reshape(-1)
    flat[blocks * 32 + lane] *= np.float32(50.0)


def gen_expert(cfg: MoEConfig, seed: int, e: int) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits of expert e's W13 [2F, D] and W2 [D, F]."""
    w13 = _rng(seed, STREAM_W13, e).standard_normal((2 * cfg.F, cfg.D), dtype=np.float32)
    w13 *= np.float32(0.02)
    w2 = _rng(seed, STREAM_W2, e).standard_normal((cfg.D, cfg.F), dtype=np.float32)
    w2 *= np.float32(0.02)
    if cfg.outliers:
        r = _rng(seed, STREAM_OUTLIER, e)
        _plant_outliers(w13, r)
        _plant_outliers(w2, r)
    return f32_to_bf16_bits(w13), f32_to_bf16_bits(w2)


def gen_experts(cfg: MoEConfig, seed: int, threads: int = 8) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits of all experts: W13 [E, 2F, D], W2 [E, D, F].  Experts are
    independent streams, so they are drawn on parallel threads (same bits)."""
    w13 = np.empty((cfg.E, 2 * cfg.F, cfg.D), dtype=np.uint16)
    w2 = np.empty((cfg.E, cfg.D, cfg.F), dtype=np.uint16)

    def one(e):
        w13[e], w2[e] = gen_expert(cfg, seed, e)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(cfg.E)))
    return w13, w2

