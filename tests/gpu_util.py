"""Helpers for the GPU parity tests (host <-> device marshalling, tolerance)."""

from __future__ import annotations

import os

import numpy as np
import torch

THREADS = int(os.environ.get("MOE_TEST_THREADS", "16"))


def device() -> torch.device:
    return torch.device("cuda:0")


def bf16_dev(a_bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on the GPU."""
    a = np.ascontiguousarray(a_bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to(device()).view(torch.bfloat16)


def bf16_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device())


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def output_tolerance(ref: np.ndarray) -> np.ndarray:
    """2^-7 * (|ref| + rms(ref)), rms over all compared outputs."""
    rms = float(np.sqrt(np.mean(ref * ref)))
    return 2.0 ** -7 * (np.abs(ref) + rms)


def assert_within_tolerance(got_bf16_bits: np.ndarray, ref: np.ndarray, what: str) -> float:
    got = bf16_bits_to_f64(got_bf16_bits)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    tol = output_tolerance(ref)
    ratio = np.abs(got - ref) / tol
    worst = float(ratio.max())
    assert worst <= 1.0, "%s: max err/tol = %.3f at %s" % (
        what, worst, np.unravel_index(int(ratio.argmax()), ratio.shape))
    return worst
