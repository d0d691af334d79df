"""Thin Python binding of libmoe_mxfp4 (MXFP4 mixture-of-experts MLP layer
for AMD MI355X / gfx950), ABI version 2.

Every step of the layer runs in the HIP kernels of libmoe_mxfp4.so; this
module only marshals torch tensors (device memory and the current stream)
into the C ABI declared in include/moe_mxfp4.h.  There is no CPU fallback: if
the library is missing, or a tensor is not on the GPU, the call raises.

Functions mirror the C entry points:
    mxfp4_quantize(w, rule)           -> (q, s)
    mxfp4_dequantize(q, s)            -> bf16 tensor
    mxfp4_pack(q)                     -> codes reordered for the expert kernels
    moe_route(x, wr, br, k)           -> Routing
    moe_expert_mlp(x, weights, routing, algo=MLP_AUTO) -> bf16 [T, D]
      (moe_expert_mlp_ex in the C ABI when an algorithm is named or the
      weights are packed)
    moe_expert_mlp_noalloc(x, weights, routing, out, algo=MLP_AUTO)
and MoELayer bundles quantized weights and workspaces for repeated calls.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = ["mxfp4_quantize", "mxfp4_dequantize", "mxfp4_pack", "moe_route", "moe_expert_mlp",
           "moe_expert_mlp_noalloc", "NOALLOC_SCRATCH_BYTES",
           "Routing", "ExpertWeights", "MoELayer", "MoEError", "lib",
           "SCALE_FLOOR_DIV6", "SCALE_OCP", "SCALE_CEIL_DIV6", "ROUND_NEAREST_EVEN",
           "ROUND_STOCHASTIC", "MLP_AUTO", "MLP_STREAM", "MLP_GROUPED_GEMM", "MLP_WEIGHTS_PACKED",
           "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mxfp4.so")
ABI_VERSION = 4
NOALLOC_SCRATCH_BYTES = 16 << 20   # MOE_NOALLOC_SCRATCH_BYTES
SCALE_FLOOR_DIV6 = 0
SCALE_OCP = 1
SCALE_CEIL_DIV6 = 2
ROUND_NEAREST_EVEN, ROUND_STOCHASTIC = 0, 1
MLP_AUTO, MLP_STREAM, MLP_GROUPED_GEMM = 0, 1, 2
MLP_WEIGHTS_PACKED = 0x100   # flag OR-ed into the algorithm: codes in mxfp4_pack's layout


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().moe_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe_mxfp4.so (built in-tree by build.py); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m mxfp4_quantized_mixture_amd.build` "
                "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        if L.moe_abi_version() != ABI_VERSION:
            raise ImportError("%s has ABI version %d, this binding needs %d: rebuild it"
                              % (LIB_PATH, L.moe_abi_version(), ABI_VERSION))
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_abi_version.argtypes = []
        L.moe_abi_version.restype = ctypes.c_int
        L.mxfp4_quantize.argtypes = [P, i64, i64, P, P, ctypes.c_int, P]
        L.mxfp4_quantize.restype = ctypes.c_int
        L.mxfp4_quantize_ex.argtypes = [P, i64, i64, P, P, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_uint64, P]
        L.mxfp4_quantize_ex.restype = ctypes.c_int
        L.mxfp4_dequantize.argtypes = [P, P, i64, i64, P, P]
        L.mxfp4_dequantize.restype = ctypes.c_int
        L.mxfp4_pack.argtypes = [P, i64, i64, P, P]
        L.mxfp4_pack.restype = ctypes.c_int
        L.moe_route_workspace_size.argtypes = [i32, i32, i32, i32]
        L.moe_route_workspace_size.restype = sz
        L.moe_route.argtypes = [P, P, P, i32, i32, i32, i32, P, P, P, P, P, P, P, P, sz, P]
        L.moe_route.restype = ctypes.c_int
        L.moe_expert_mlp_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.moe_expert_mlp_workspace_size.restype = sz
        L.moe_expert_mlp.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                     P, P, sz, P]
        L.moe_expert_mlp.restype = ctypes.c_int
        L.moe_expert_mlp_ex.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                        P, P, sz, ctypes.c_int, P, P]
        L.moe_expert_mlp_ex.restype = ctypes.c_int
        L.moe_expert_mlp_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                             P, ctypes.c_int, P]
        L.moe_expert_mlp_noalloc.restype = ctypes.c_int
        L.moe_expert_mlp_bf16_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.moe_expert_mlp_bf16_workspace_size.restype = sz
        L.moe_expert_mlp_bf16.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                          P, P, sz, P]
        L.moe_expert_mlp_bf16.restype = ctypes.c_int
        L.moe_expert_mlp_bf16_ex.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                             P, P, sz, P, P]
        L.moe_expert_mlp_bf16_ex.restype = ctypes.c_int
        L.moe_layer_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.moe_layer_decode_workspace_size.restype = sz
        L.moe_layer_decode_init.argtypes = [P, sz, P]
        L.moe_layer_decode_init.restype = ctypes.c_int
        L.moe_layer_decode.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                       P, P, P, P, P, P, P, P, sz, ctypes.c_int, P]
        L.moe_layer_decode.restype = ctypes.c_int
        L.moe_layer_decode_ex.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                          P, P, P, P, P, P, P, P, sz, ctypes.c_int, i32, P, P]
        L.moe_layer_decode_ex.restype = ctypes.c_int
        L.moe_layer_decode_error.argtypes = [P, P, P]
        L.moe_layer_decode_error.restype = ctypes.c_int
        _lib = L
    return _lib


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoEError(fn, status)


# ---------------------------------------------------------------- codec

def mxfp4_quantize(w: torch.Tensor, rule: int = SCALE_FLOOR_DIV6, stochastic: bool = False,
                   seed: int = 0):
    """bf16 [..., K] -> (codes uint8 [..., K/2], E8M0 scales uint8 [..., K/32]).
    stochastic: stochastic rounding drawn from the SplitMix64 stream of `seed`."""
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    q = torch.empty(*w.shape[:-1], K // 2, dtype=torch.uint8, device=w.device)
    s = torch.empty(*w.shape[:-1], K // 32, dtype=torch.uint8, device=w.device)
    _check("mxfp4_quantize", lib().mxfp4_quantize_ex(
        _dev(w, "w", torch.bfloat16), rows, K, _dev(q, "q"), _dev(s, "s"), rule,
        ROUND_STOCHASTIC if stochastic else ROUND_NEAREST_EVEN, int(seed) & (2**64 - 1),
        _stream(w.device)))
    return q, s


def mxfp4_dequantize(q: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    K = q.shape[-1] * 2
    rows = q.numel() // q.shape[-1]
    out = torch.empty(*q.shape[:-1], K, dtype=torch.bfloat16, device=q.device)
    _check("mxfp4_dequantize", lib().mxfp4_dequantize(
        _dev(q, "q", torch.uint8), _dev(s, "s", torch.uint8), rows, K, _dev(out, "out"),
        _stream(q.device)))
    return out


def mxfp4_pack(q: torch.Tensor) -> torch.Tensor:
    """Codes uint8 [..., K/2] (rows a multiple of 32, K % 64 == 0) -> the same
    codes with each 32-row x 64-element fragment contiguous (1 KiB: the first
    32-element halves of its 32 rows, then the second halves), fragments in
    (row group, contraction step) order.  The scales keep their layout."""
    K = q.shape[-1] * 2
    rows = q.numel() // q.shape[-1] if q.shape[-1] else 0
    out = torch.empty_like(q)
    _check("mxfp4_pack", lib().mxfp4_pack(_dev(q, "q", torch.uint8), rows, K, _dev(out, "out"),
                                          _stream(q.device)))
    return out


# ---------------------------------------------------------------- routing

@dataclass
class Routing:
    ids: torch.Tensor        # int32 [T, k]
    weights: torch.Tensor    # fp32 [T, k]
    counts: torch.Tensor     # int32 [E]
    offsets: torch.Tensor    # int32 [E+1]
    sorted_pairs: torch.Tensor  # int32 [T*k]
    pair_pos: torch.Tensor   # int32 [T*k]
    logits: torch.Tensor | None = None  # fp32 [T, E]


def alloc_routing(T: int, E: int, k: int, device, with_logits: bool = False) -> Routing:
    i32 = dict(dtype=torch.int32, device=device)
    return Routing(
        ids=torch.empty(T, k, **i32), weights=torch.empty(T, k, dtype=torch.float32, device=device),
        counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
        sorted_pairs=torch.empty(T * k, **i32), pair_pos=torch.empty(T * k, **i32),
        logits=torch.empty(T, E, dtype=torch.float32, device=device) if with_logits else None)


def route_workspace(T: int, D: int, E: int, k: int, device) -> torch.Tensor:
    n = lib().moe_route_workspace_size(T, D, E, k)
    if n == 0:
        raise MoEError("moe_route_workspace_size", 2)
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_route(x: torch.Tensor, wr: torch.Tensor, br: torch.Tensor | None, k: int,
              out: Routing | None = None, ws: torch.Tensor | None = None,
              with_logits: bool = False) -> Routing:
    T, D = x.shape
    E = wr.shape[0]
    if wr.shape[1] != D:
        raise ValueError("router weight must be [E, D]")
    r = out if out is not None else alloc_routing(T, E, k, x.device, with_logits)
    ws = ws if ws is not None else route_workspace(T, D, E, k, x.device)
    _check("moe_route", lib().moe_route(
        _dev(x, "x", torch.bfloat16), _dev(wr, "wr", torch.float32),
        None if br is None else _dev(br, "br", torch.float32), T, D, E, k,
        _dev(r.ids, "ids"), _dev(r.weights, "weights"), _dev(r.counts, "counts"),
        _dev(r.offsets, "offsets"), _dev(r.sorted_pairs, "sorted_pairs"),
        _dev(r.pair_pos, "pair_pos"), None if r.logits is None else _dev(r.logits, "logits"),
        _dev(ws, "ws"), ws.numel(), _stream(x.device)))
    return r


# ---------------------------------------------------------------- experts

@dataclass
class ExpertWeights:
    w13_q: torch.Tensor   # uint8 [E, 2F, D/2]
    w13_s: torch.Tensor   # uint8 [E, 2F, D/32]
    w2_q: torch.Tensor    # uint8 [E, D, F/2]
    w2_s: torch.Tensor    # uint8 [E, D, F/32]
    packed: bool = False  # codes (w13_q, w2_q) in mxfp4_pack's layout

    @property
    def E(self) -> int:
        return self.w13_q.shape[0]

    @property
    def F(self) -> int:
        return self.w2_q.shape[2] * 2

    @property
    def D(self) -> int:
        return self.w2_q.shape[1]

    @property
    def algo_flags(self) -> int:
        return MLP_WEIGHTS_PACKED if self.packed else 0

    def pack(self) -> "ExpertWeights":
        """The same weights with the codes in mxfp4_pack's layout."""
        if self.packed:
            return self
        return ExpertWeights(mxfp4_pack(self.w13_q), self.w13_s, mxfp4_pack(self.w2_q),
                             self.w2_s, True)

    @classmethod
    def quantize(cls, w13: torch.Tensor, w2: torch.Tensor, rule: int = SCALE_FLOOR_DIV6,
                 packed: bool = False):
        """bf16 W13 [E, 2F, D] and W2 [E, D, F] -> MXFP4 (codes packed on request)."""
        a, b = mxfp4_quantize(w13, rule)
        c, d = mxfp4_quantize(w2, rule)
        w = cls(a, b, c, d)
        return w.pack() if packed else w


def _event_array(events) -> ctypes.Array:
    """4 torch.cuda.Event objects -> hipEvent_t[4].  torch creates the native
    event lazily, on its first record(), so record each once if needed."""
    if len(events) != 4:
        raise ValueError("events must hold 4 torch.cuda.Event objects")
    for e in events:
        if not e.cuda_event:
            e.record()
    return (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])


def mlp_workspace(T: int, D: int, F: int, E: int, k: int, device) -> torch.Tensor:
    n = lib().moe_expert_mlp_workspace_size(T, D, F, E, k)
    if n == 0:
        raise MoEError("moe_expert_mlp_workspace_size", 2)
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_expert_mlp(x: torch.Tensor, weights: ExpertWeights, routing: Routing,
                   out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                   events=None, algo: int = MLP_AUTO) -> torch.Tensor:
    T, D = x.shape
    E, F = weights.E, weights.F
    k = routing.ids.shape[1]
    if weights.D != D:
        raise ValueError("expert weights do not match d_model")
    out = out if out is not None else torch.empty(T, D, dtype=torch.bfloat16, device=x.device)
    ws = ws if ws is not None else mlp_workspace(T, D, F, E, k, x.device)
    ev = None if events is None else _event_array(events)
    _check("moe_expert_mlp", lib().moe_expert_mlp_ex(
        _dev(x, "x", torch.bfloat16), _dev(weights.w13_q, "w13_q", torch.uint8),
        _dev(weights.w13_s, "w13_s", torch.uint8), _dev(weights.w2_q, "w2_q", torch.uint8),
        _dev(weights.w2_s, "w2_s", torch.uint8), _dev(routing.weights, "topk_w", torch.float32),
        _dev(routing.offsets, "offsets", torch.int32),
        _dev(routing.sorted_pairs, "sorted_pairs", torch.int32),
        _dev(routing.pair_pos, "pair_pos", torch.int32), T, D, F, E, k,
        _dev(out, "out", torch.bfloat16), _dev(ws, "ws"), ws.numel(), algo | weights.algo_flags,
        ev, _stream(x.device)))
    return out


def moe_expert_mlp_noalloc(x: torch.Tensor, weights: ExpertWeights, routing: Routing,
                           out: torch.Tensor, algo: int = MLP_AUTO) -> torch.Tensor:
    """moe_expert_mlp on the library's fixed per-GPU workspace (no workspace
    argument; nothing is allocated, `out` must be given).  Calls that overlap
    on one GPU race on that workspace."""
    T, D = x.shape
    E, F = weights.E, weights.F
    k = routing.ids.shape[1]
    if weights.D != D:
        raise ValueError("expert weights do not match d_model")
    _check("moe_expert_mlp_noalloc", lib().moe_expert_mlp_noalloc(
        _dev(x, "x", torch.bfloat16), _dev(weights.w13_q, "w13_q", torch.uint8),
        _dev(weights.w13_s, "w13_s", torch.uint8), _dev(weights.w2_q, "w2_q", torch.uint8),
        _dev(weights.w2_s, "w2_s", torch.uint8), _dev(routing.weights, "topk_w", torch.float32),
        _dev(routing.offsets, "offsets", torch.int32),
        _dev(routing.sorted_pairs, "sorted_pairs", torch.int32),
        _dev(routing.pair_pos, "pair_pos", torch.int32), T, D, F, E, k,
        _dev(out, "out", torch.bfloat16), algo | weights.algo_flags, _stream(x.device)))
    return out


def mlp_bf16_workspace(T: int, D: int, F: int, E: int, k: int, device) -> torch.Tensor:
    n = lib().moe_expert_mlp_bf16_workspace_size(T, D, F, E, k)
    if n == 0:
        raise MoEError("moe_expert_mlp_bf16_workspace_size", 2)
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_expert_mlp_bf16(x: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, routing: Routing,
                        out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                        events=None) -> torch.Tensor:
    """The expert layer on bf16 weights: w13 [E, 2F, D], w2 [E, D, F] (the
    comparison path of the MXFP4 one; same routing and output)."""
    T, D = x.shape
    E, F2, D13 = w13.shape
    F = F2 // 2
    k = routing.ids.shape[1]
    if D13 != D or F2 != 2 * F or tuple(w2.shape) != (E, D, F):
        raise ValueError("bf16 expert weights must be [E, 2F, D] and [E, D, F]")
    out = out if out is not None else torch.empty(T, D, dtype=torch.bfloat16, device=x.device)
    ws = ws if ws is not None else mlp_bf16_workspace(T, D, F, E, k, x.device)
    ev = None if events is None else _event_array(events)
    _check("moe_expert_mlp_bf16", lib().moe_expert_mlp_bf16_ex(
        _dev(x, "x", torch.bfloat16), _dev(w13, "w13", torch.bfloat16),
        _dev(w2, "w2", torch.bfloat16), _dev(routing.weights, "topk_w", torch.float32),
        _dev(routing.offsets, "offsets", torch.int32),
        _dev(routing.sorted_pairs, "sorted_pairs", torch.int32),
        _dev(routing.pair_pos, "pair_pos", torch.int32), T, D, F, E, k,
        _dev(out, "out", torch.bfloat16), _dev(ws, "ws"), ws.numel(), ev, _stream(x.device)))
    return out


DECODE_SPIN_LIMIT = 1 << 20


def decode_workspace(T: int, D: int, F: int, E: int, k: int, device) -> torch.Tensor:
    """Workspace of moe_layer_decode, its control block initialised."""
    n = lib().moe_layer_decode_workspace_size(T, D, F, E, k)
    if n == 0:
        raise MoEError("moe_layer_decode_workspace_size", 2)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    decode_init(ws)
    return ws


def decode_init(ws: torch.Tensor) -> None:
    _check("moe_layer_decode_init", lib().moe_layer_decode_init(
        _dev(ws, "ws"), ws.numel(), _stream(ws.device)))


def decode_error(ws: torch.Tensor) -> int:
    """The control block's error word (waits for the current stream)."""
    v = ctypes.c_int32(-1)
    _check("moe_layer_decode_error", lib().moe_layer_decode_error(
        _dev(ws, "ws"), ctypes.byref(v), _stream(ws.device)))
    return v.value


def moe_layer_decode(x: torch.Tensor, wr: torch.Tensor, br: torch.Tensor | None,
                     weights: ExpertWeights, k: int, out: torch.Tensor | None = None,
                     routing: Routing | None = None, ws: torch.Tensor | None = None,
                     events=None, spin_limit: int = DECODE_SPIN_LIMIT):
    """Route + experts of a decode-sized batch with the routing fused into the
    gate/up weight stream.  Returns (out, routing)."""
    T, D = x.shape
    E, F = weights.E, weights.F
    if weights.D != D:
        raise ValueError("expert weights do not match d_model")
    out = out if out is not None else torch.empty(T, D, dtype=torch.bfloat16, device=x.device)
    r = routing if routing is not None else alloc_routing(T, E, k, x.device)
    ws = ws if ws is not None else decode_workspace(T, D, F, E, k, x.device)
    ev = None if events is None else _event_array(events)
    _check("moe_layer_decode", lib().moe_layer_decode_ex(
        _dev(x, "x", torch.bfloat16), _dev(wr, "wr", torch.float32),
        None if br is None else _dev(br, "br", torch.float32),
        _dev(weights.w13_q, "w13_q", torch.uint8), _dev(weights.w13_s, "w13_s", torch.uint8),
        _dev(weights.w2_q, "w2_q", torch.uint8), _dev(weights.w2_s, "w2_s", torch.uint8),
        T, D, F, E, k, _dev(r.ids, "ids"), _dev(r.weights, "weights"), _dev(r.counts, "counts"),
        _dev(r.offsets, "offsets"), _dev(r.sorted_pairs, "sorted_pairs"),
        _dev(r.pair_pos, "pair_pos"), _dev(out, "out", torch.bfloat16), _dev(ws, "ws"),
        ws.numel(), weights.algo_flags, spin_limit, ev, _stream(x.device)))
    return out, r


class PreparedDecodeLayer:
    """moe_layer_decode with every C-ABI argument marshalled once (the
    decode counterpart of PreparedLayer: calling it re-issues one C call)."""

    def __init__(self, x: torch.Tensor, wr: torch.Tensor, br: torch.Tensor | None,
                 weights: ExpertWeights, k: int, out: torch.Tensor, routing: Routing,
                 ws: torch.Tensor, stream=None):
        T, D = x.shape
        E, F = weights.E, weights.F
        self.L = lib()
        st = (stream or torch.cuda.current_stream(x.device)).cuda_stream
        self._keep = (x, wr, br, weights, out, routing, ws)
        self.head = (
            _dev(x, "x", torch.bfloat16), _dev(wr, "wr", torch.float32),
            None if br is None else _dev(br, "br", torch.float32),
            _dev(weights.w13_q, "w13_q", torch.uint8), _dev(weights.w13_s, "w13_s", torch.uint8),
            _dev(weights.w2_q, "w2_q", torch.uint8), _dev(weights.w2_s, "w2_s", torch.uint8),
            T, D, F, E, k, _dev(routing.ids, "ids"), _dev(routing.weights, "weights"),
            _dev(routing.counts, "counts"), _dev(routing.offsets, "offsets"),
            _dev(routing.sorted_pairs, "sorted_pairs"), _dev(routing.pair_pos, "pair_pos"),
            _dev(out, "out", torch.bfloat16), _dev(ws, "ws"), ws.numel(), weights.algo_flags,
            DECODE_SPIN_LIMIT)
        self.stream = st

    @staticmethod
    def event_array(events) -> ctypes.Array:
        return _event_array(events)

    def __call__(self, event_array=None) -> None:
        s = self.L.moe_layer_decode_ex(*self.head, event_array, self.stream)
        if s:
            raise MoEError("moe_layer_decode", s)


class MoELayer:
    """Router + MXFP4 experts with preallocated routing buffers and workspaces."""

    def __init__(self, wr: torch.Tensor, br: torch.Tensor | None, weights: ExpertWeights,
                 k: int, max_tokens: int):
        self.wr, self.br, self.weights, self.k = wr, br, weights, k
        self.max_tokens = max_tokens
        dev = wr.device
        E, D, F = weights.E, weights.D, weights.F
        self.routing = alloc_routing(max_tokens, E, k, dev)
        self.route_ws = route_workspace(max_tokens, D, E, k, dev)
        self.mlp_ws = mlp_workspace(max_tokens, D, F, E, k, dev)

    def __call__(self, x: torch.Tensor, out: torch.Tensor | None = None, events=None):
        T = x.shape[0]
        if T != self.max_tokens:
            raise ValueError("MoELayer was sized for %d tokens" % self.max_tokens)
        r = moe_route(x, self.wr, self.br, self.k, out=self.routing, ws=self.route_ws)
        return moe_expert_mlp(x, self.weights, r, out=out, ws=self.mlp_ws, events=events)


class PreparedLayer:
    """Route + experts with every C-ABI argument marshalled once.

    For tight loops (decode steps): calling it only re-issues the two C calls
    on the stream captured at construction, so the host adds no per-call
    tensor checks.  Buffers must stay alive and unchanged in shape.
    """

    def __init__(self, x: torch.Tensor, wr: torch.Tensor, br: torch.Tensor | None,
                 weights, k: int, out: torch.Tensor, routing: Routing,
                 route_ws: torch.Tensor, mlp_ws: torch.Tensor, stream=None,
                 algo: int = MLP_AUTO):
        """weights: ExpertWeights (MXFP4, moe_expert_mlp_ex), or a (w13, w2)
        pair of bf16 tensors [E, 2F, D], [E, D, F] (moe_expert_mlp_bf16_ex)."""
        T, D = x.shape
        self.L = lib()
        st = (stream or torch.cuda.current_stream(x.device)).cuda_stream
        self._keep = (x, wr, br, weights, out, routing, route_ws, mlp_ws)
        self.bf16 = not isinstance(weights, ExpertWeights)
        if self.bf16:
            w13, w2 = weights
            E, F = w13.shape[0], w13.shape[1] // 2
            if tuple(w13.shape) != (E, 2 * F, D) or tuple(w2.shape) != (E, D, F):
                raise ValueError("bf16 expert weights must be [E, 2F, D] and [E, D, F]")
        else:
            E, F = weights.E, weights.F
        self.route_args = (
            _dev(x, "x", torch.bfloat16), _dev(wr, "wr", torch.float32),
            None if br is None else _dev(br, "br", torch.float32), T, D, E, k,
            _dev(routing.ids, "ids"), _dev(routing.weights, "weights"),
            _dev(routing.counts, "counts"), _dev(routing.offsets, "offsets"),
            _dev(routing.sorted_pairs, "sorted_pairs"), _dev(routing.pair_pos, "pair_pos"),
            None, _dev(route_ws, "ws"), route_ws.numel(), st)
        tail = (_dev(routing.weights, "topk_w"), _dev(routing.offsets, "offsets"),
                _dev(routing.sorted_pairs, "sorted_pairs"), _dev(routing.pair_pos, "pair_pos"),
                T, D, F, E, k, _dev(out, "out", torch.bfloat16), _dev(mlp_ws, "ws"),
                mlp_ws.numel())
        if self.bf16:
            self.mlp_head = (_dev(x, "x", torch.bfloat16), _dev(w13, "w13", torch.bfloat16),
                             _dev(w2, "w2", torch.bfloat16)) + tail
        else:
            self.mlp_head = (
                _dev(x, "x", torch.bfloat16), _dev(weights.w13_q, "w13_q", torch.uint8),
                _dev(weights.w13_s, "w13_s", torch.uint8), _dev(weights.w2_q, "w2_q", torch.uint8),
                _dev(weights.w2_s, "w2_s", torch.uint8)) + tail + (algo | weights.algo_flags,)
        self.stream = st

    @staticmethod
    def event_array(events) -> ctypes.Array:
        return _event_array(events)

    def __call__(self, event_array=None) -> None:
        s = self.L.moe_route(*self.route_args)
        if s:
            raise MoEError("moe_route", s)
        if self.bf16:
            s = self.L.moe_expert_mlp_bf16_ex(*self.mlp_head, event_array, self.stream)
        else:
            s = self.L.moe_expert_mlp_ex(*self.mlp_head, event_array, self.stream)
        if s:
            raise MoEError("moe_expert_mlp_bf16" if self.bf16 else "moe_expert_mlp", s)
