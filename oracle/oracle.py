"""ctypes front end of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check in
__graft_entry__.py and by the cpu_baseline leg of bench.py, never by the
product package.  It shares no code with the HIP library.

All arrays are NumPy; bf16 values travel as their uint16 bit patterns.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = f64
        L.oracle_e2m1_value.argtypes = [i32]
        L.oracle_e2m1_value.restype = f64
        L.oracle_e8m0_value.argtypes = [i32]
        L.oracle_e8m0_value.restype = f64
        L.oracle_scale_exponent.argtypes = [f64, i32]
        L.oracle_scale_exponent.restype = i32
        L.oracle_e2m1_encode.argtypes = [f64]
        L.oracle_e2m1_encode.restype = i32
        L.oracle_quantize.argtypes = [P, i64, i64, i32, P, P]
        L.oracle_quantize.restype = i32
        L.oracle_quantize_ex.argtypes = [P, i64, i64, i32, i32, ctypes.c_uint64, P, P]
        L.oracle_quantize_ex.restype = i32
        L.oracle_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.oracle_splitmix64.restype = ctypes.c_uint64
        L.oracle_e2m1_encode_stochastic.argtypes = [f64, ctypes.c_uint32]
        L.oracle_e2m1_encode_stochastic.restype = i32
        L.oracle_dequantize.argtypes = [P, P, i64, i64, P]
        L.oracle_dequantize.restype = None
        L.oracle_route.argtypes = [P, P, P, i32, i32, i32, i32,
                                   P, P, P, P, P, P, P, P]
        L.oracle_route.restype = i32
        L.oracle_moe.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                 P, i32, P]
        L.oracle_moe.restype = i32
        L.oracle_expert_mlp.argtypes = [P, i32, i32, P, P, P, P, P, i32, P]
        L.oracle_expert_mlp.restype = i32
        L.oracle_expert_mlp_bf16.argtypes = [P, i32, i32, P, P, P, i32, P]
        L.oracle_expert_mlp_bf16.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# -- scalars ---------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def e8m0_value(byte: int) -> float:
    return lib().oracle_e8m0_value(int(byte))


def scale_exponent(amax: float, rule: int = 0) -> int:
    return lib().oracle_scale_exponent(float(amax), int(rule))


def e2m1_encode(y: float) -> int:
    return lib().oracle_e2m1_encode(float(y))


def e2m1_encode_stochastic(y: float, u: int) -> int:
    """Stochastic E2M1 code of an already-scaled y with the 24-bit draw u."""
    return lib().oracle_e2m1_encode_stochastic(float(y), int(u))


def splitmix64(seed: int, n: int) -> int:
    """Output n >= 1 of the SplitMix64 generator whose state starts at seed."""
    return lib().oracle_splitmix64(int(seed) & (2**64 - 1), int(n) & (2**64 - 1))


# -- MXFP4 -----------------------------------------------------------------

def quantize(w_bf16: np.ndarray, rule: int = 0, stochastic: bool = False,
             seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits [..., K] -> (packed codes [..., K/2], E8M0 scales [..., K/32]).
    stochastic: stochastic rounding with the SplitMix64 stream of `seed`."""
    w = _c(w_bf16, np.uint16)
    K = w.shape[-1]
    rows = w.size // K
    q = np.empty(w.shape[:-1] + (K // 2,), dtype=np.uint8)
    s = np.empty(w.shape[:-1] + (K // 32,), dtype=np.uint8)
    rc = lib().oracle_quantize_ex(_ptr(w), rows, K, rule, 1 if stochastic else 0,
                                  int(seed) & (2**64 - 1), _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("oracle_quantize rejected its arguments (rc=%d)" % rc)
    return q, s


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    K = q.shape[-1] * 2
    rows = q.size // q.shape[-1]
    out = np.empty(q.shape[:-1] + (K,), dtype=np.float64)
    lib().oracle_dequantize(_ptr(q), _ptr(s), rows, K, _ptr(out))
    return out


# -- routing ---------------------------------------------------------------

def route(x_bf16: np.ndarray, wr: np.ndarray, b: np.ndarray | None, k: int) -> dict:
    x = _c(x_bf16, np.uint16)
    wr = _c(wr, np.float32)
    T, D = x.shape
    E = wr.shape[0]
    bb = None if b is None else _c(b, np.float32)
    out = dict(
        logits=np.empty((T, E), np.float64), ids=np.empty((T, k), np.int32),
        w=np.empty((T, k), np.float64), gap=np.empty(T, np.float64),
        counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
        sorted=np.empty(T * k, np.int32), pos=np.empty(T * k, np.int32))
    rc = lib().oracle_route(_ptr(x), _ptr(wr), _ptr(bb), T, D, E, k,
                            _ptr(out["logits"]), _ptr(out["ids"]), _ptr(out["w"]),
                            _ptr(out["gap"]), _ptr(out["counts"]), _ptr(out["offsets"]),
                            _ptr(out["sorted"]), _ptr(out["pos"]))
    if rc != 0:
        raise ValueError("oracle_route rejected its arguments (rc=%d)" % rc)
    return out


# -- expert MLP + combine ----------------------------------------------------

def moe(x_bf16, q13, s13, q2, s2, ids, w, F: int, tokens=None) -> np.ndarray:
    """fp64 layer output for the listed tokens (all tokens if None): [n, D]."""
    x = _c(x_bf16, np.uint16)
    T, D = x.shape
    q13, s13, q2, s2 = (_c(a, np.uint8) for a in (q13, s13, q2, s2))
    E = q13.shape[0]
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    k = ids.shape[1]
    toks = None if tokens is None else _c(tokens, np.int32)
    n = T if toks is None else len(toks)
    out = np.empty((n, D), np.float64)
    rc = lib().oracle_moe(_ptr(x), _ptr(q13), _ptr(s13), _ptr(q2), _ptr(s2),
                          _ptr(ids), _ptr(w), T, D, F, E, k, _ptr(toks), n, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_moe failed (rc=%d)" % rc)
    return out


def expert_mlp(x_bf16, q13e, s13e, q2e, s2e, F: int, tokens) -> np.ndarray:
    """One expert on the listed tokens: y [n, D] fp64 (see oracle_expert_mlp)."""
    x = _c(x_bf16, np.uint16)
    D = x.shape[1]
    q13e, s13e, q2e, s2e = (_c(a, np.uint8) for a in (q13e, s13e, q2e, s2e))
    toks = _c(tokens, np.int32)
    y = np.empty((len(toks), D), np.float64)
    rc = lib().oracle_expert_mlp(_ptr(x), D, F, _ptr(q13e), _ptr(s13e), _ptr(q2e), _ptr(s2e),
                                 _ptr(toks), len(toks), _ptr(y))
    if rc != 0:
        raise ValueError("oracle_expert_mlp failed (rc=%d)" % rc)
    return y


def expert_mlp_bf16(x_bf16, w13e, w2e, F: int, tokens) -> np.ndarray:
    """One expert with bf16 weights (w13e [2F, D], w2e [D, F] as bf16 bit
    patterns) on the listed tokens: y [n, D] fp64 (see oracle_expert_mlp_bf16)."""
    x = _c(x_bf16, np.uint16)
    D = x.shape[1]
    w13e, w2e = _c(w13e, np.uint16), _c(w2e, np.uint16)
    if w13e.shape != (2 * F, D) or w2e.shape != (D, F):
        raise ValueError("bf16 expert weights must be [2F, D] and [D, F]")
    toks = _c(tokens, np.int32)
    y = np.empty((len(toks), D), np.float64)
    rc = lib().oracle_expert_mlp_bf16(_ptr(x), D, F, _ptr(w13e), _ptr(w2e), _ptr(toks),
                                      len(toks), _ptr(y))
    if rc != 0:
        raise ValueError("oracle_expert_mlp_bf16 failed (rc=%d)" % rc)
    return y


def moe_threaded(x_bf16, expert_weights, ids, w, F: int, tokens=None, threads: int = 8):
    """Same result as moe(), with experts evaluated on parallel threads.

    expert_weights(e) returns expert e's weights (so experts can be prepared
    lazily, on the worker threads): either its MXFP4 arrays (q13e, s13e, q2e,
    s2e), evaluated by oracle_expert_mlp, or its bf16 matrices (w13e, w2e),
    evaluated by oracle_expert_mlp_bf16.  Each worker runs the single-threaded
    oracle; the slot-order combine out[t] = sum_j w[t, j] * y(t, j) is then
    done here in fp64, j ascending.
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    D = np.asarray(x_bf16).shape[1]
    y = np.zeros((len(toks), k, D), np.float64)
    jobs = {}
    for i, t in enumerate(toks):
        for j in range(k):
            jobs.setdefault(int(ids[t, j]), []).append((i, j, int(t)))

    def run(e):
        we = expert_weights(e)
        lst = jobs[e]
        tl = [t for _, _, t in lst]
        if len(we) == 2:
            ye = expert_mlp_bf16(x_bf16, we[0], we[1], F, tl)
        else:
            ye = expert_mlp(x_bf16, *we, F, tl)
        for r, (i, j, _) in enumerate(lst):
            y[i, j] = ye[r]

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, sorted(jobs)))
    w = np.asarray(w, np.float64)
    out = np.zeros((len(toks), D), np.float64)
    for j in range(k):
        out = out + w[toks, j][:, None] * y[:, j, :]
    return out
