"""The C ABI library loads, exports every symbol the header declares, and
rejects bad arguments before enqueuing anything (no GPU needed: every call
here fails validation on the host)."""

import ctypes
import os
import re

import pytest

import mxfp4_quantized_mixture_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")

OK, NULL, SHAPE, WS, ENUM, HIP, ALIGN = range(7)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from mxfp4_quantized_mixture_amd import build
        build.build()
    return moe.lib()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"MOE_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"mxfp4_quantize", "mxfp4_quantize_ex", "mxfp4_pack", "moe_route", "moe_expert_mlp",
            "moe_route_workspace_size",
            "moe_expert_mlp_workspace_size", "moe_status_string", "mxfp4_dequantize",
            "moe_abi_version"} <= names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_no_internal_symbols_exported():
    out = os.popen("nm -D --defined-only %s" % moe.LIB_PATH).read()
    text_syms = [l.split()[-1] for l in out.splitlines() if " T " in l]
    assert set(text_syms) == set(declared_functions())


def test_status_strings(L):
    assert L.moe_status_string(OK) == b"ok"
    for s in range(1, 7):
        assert L.moe_status_string(s) and L.moe_status_string(s) != b"ok"
    assert L.moe_abi_version() == 1


def test_workspace_sizes(L):
    assert L.moe_route_workspace_size(32, 2880, 32, 4) > 0
    assert L.moe_expert_mlp_workspace_size(32, 2880, 2880, 32, 4) >= 32 * 4 * 2880 * 6
    assert L.moe_route_workspace_size(0, 2880, 32, 4) == 0        # T < 1
    assert L.moe_route_workspace_size(8, 2880, 4, 5) == 0         # k > E
    assert L.moe_route_workspace_size(8, 2880, 300, 4) == 0       # E > 256
    assert L.moe_route_workspace_size(8, 2880, 32, 9) == 0        # k > 8
    assert L.moe_route_workspace_size(8, 100, 32, 4) == 0         # D % 32
    assert L.moe_expert_mlp_workspace_size(8, 64, 48, 4, 2) == 0  # F % 32


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def test_quantize_validation(L):
    assert L.mxfp4_quantize(FAKE, 4, 48, 0, FAKE, FAKE, None) == SHAPE
    assert L.mxfp4_quantize(FAKE, -1, 64, 0, FAKE, FAKE, None) == SHAPE
    assert L.mxfp4_quantize(FAKE, 4, 64, 3, FAKE, FAKE, None) == ENUM
    L.mxfp4_quantize_ex.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert L.mxfp4_quantize_ex(FAKE, 4, 64, 2, 2, 0, FAKE, FAKE, None) == ENUM   # rounding
    assert L.mxfp4_quantize_ex(FAKE, 4, 64, 3, 1, 0, FAKE, FAKE, None) == ENUM   # rule
    assert L.mxfp4_quantize_ex(FAKE, 4, 48, 2, 1, 0, FAKE, FAKE, None) == SHAPE
    assert L.mxfp4_quantize_ex(None, 4, 64, 2, 1, 0, FAKE, FAKE, None) == NULL
    assert L.mxfp4_quantize_ex(None, 0, 64, 2, 1, 0, None, None, None) == OK
    assert L.mxfp4_quantize(None, 4, 64, 0, FAKE, FAKE, None) == NULL
    assert L.mxfp4_quantize(FAKE + 2, 4, 64, 0, FAKE, FAKE, None) == ALIGN
    assert L.mxfp4_quantize(None, 0, 64, 0, None, None, None) == OK    # empty: nothing to do
    assert L.mxfp4_dequantize(FAKE, FAKE, 4, 40, FAKE, None) == SHAPE
    assert L.mxfp4_dequantize(FAKE, None, 4, 64, FAKE, None) == NULL


def test_pack_validation(L):
    assert L.mxfp4_pack(FAKE, 48, 64, FAKE + 4096, None) == SHAPE        # rows % 32
    assert L.mxfp4_pack(FAKE, 32, 96, FAKE + 4096, None) == SHAPE        # K % 64
    assert L.mxfp4_pack(FAKE, -32, 64, FAKE + 4096, None) == SHAPE
    assert L.mxfp4_pack(None, 32, 64, FAKE, None) == NULL
    assert L.mxfp4_pack(FAKE + 8, 32, 64, FAKE + 4096, None) == ALIGN
    assert L.mxfp4_pack(FAKE, 32, 64, FAKE, None) == SHAPE               # in place
    assert L.mxfp4_pack(FAKE, 32, 64, FAKE + 512, None) == SHAPE         # overlapping
    assert L.mxfp4_pack(None, 0, 64, None, None) == OK


def _route(L, T=8, D=64, E=4, k=2, x=FAKE, ws=FAKE, ws_bytes=None, null_out=False):
    if ws_bytes is None:
        ws_bytes = L.moe_route_workspace_size(T, D, E, k) or 1 << 20
    o = None if null_out else FAKE
    return L.moe_route(x, FAKE, None, T, D, E, k, o, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws,
                       ws_bytes, None)


def test_route_validation(L):
    assert _route(L, T=0) == SHAPE
    assert _route(L, D=48) == SHAPE
    assert _route(L, E=0) == SHAPE
    assert _route(L, k=5, E=4) == SHAPE
    assert _route(L, x=None) == NULL
    assert _route(L, null_out=True) == NULL
    assert _route(L, ws=None) == WS
    assert _route(L, ws_bytes=16) == WS
    assert _route(L, x=FAKE + 8) == ALIGN


def _mlp(L, T=8, D=64, F=64, E=4, k=2, out=FAKE, ws_bytes=None, w13=FAKE):
    if ws_bytes is None:
        ws_bytes = L.moe_expert_mlp_workspace_size(T, D, F, E, k) or 1 << 20
    return L.moe_expert_mlp(FAKE, w13, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T, D, F, E, k,
                            out, FAKE, ws_bytes, None, None)


def test_mlp_validation(L):
    assert _mlp(L, F=40) == SHAPE
    assert _mlp(L, T=0) == SHAPE
    assert _mlp(L, out=None) == NULL
    assert _mlp(L, ws_bytes=100) == WS
    assert _mlp(L, w13=FAKE + 4) == ALIGN


def _mlp_ex(L, algo, T=8, D=64, F=64, E=4, k=2, out=FAKE):
    ws_bytes = L.moe_expert_mlp_workspace_size(T, D, F, E, k) or 1 << 20
    return L.moe_expert_mlp_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T, D, F,
                               E, k, out, FAKE, ws_bytes, algo, None, None)


def test_mlp_algorithm_validation(L):
    assert _mlp_ex(L, 3) == ENUM
    assert _mlp_ex(L, -1) == ENUM
    assert _mlp_ex(L, moe.MLP_GROUPED_GEMM, D=96) == SHAPE      # grouped GEMM needs D % 64
    assert _mlp_ex(L, moe.MLP_GROUPED_GEMM, F=160) == SHAPE     # ... and F % 64
    assert _mlp_ex(L, moe.MLP_GROUPED_GEMM, F=7296) == SHAPE    # down GEMM's LDS budget
    assert _mlp_ex(L, moe.MLP_GROUPED_GEMM, D=8256) == SHAPE    # contraction limit
    assert _mlp_ex(L, moe.MLP_STREAM, F=7296, out=None) == NULL # streaming takes any F
    assert _mlp_ex(L, moe.MLP_STREAM, out=None) == NULL
    assert _mlp_ex(L, moe.MLP_GROUPED_GEMM, out=None) == NULL
    P = moe.MLP_WEIGHTS_PACKED
    assert _mlp_ex(L, 0x200) == ENUM                                    # unknown flag
    assert _mlp_ex(L, 3 | P) == ENUM
    assert _mlp_ex(L, moe.MLP_STREAM | P, F=160) == SHAPE               # packed needs F % 64
    assert _mlp_ex(L, moe.MLP_AUTO | P, D=96) == SHAPE                  # ... and D % 64
    assert _mlp_ex(L, moe.MLP_STREAM | P, D=3904) == SHAPE              # streaming LDS budget
    assert _mlp_ex(L, moe.MLP_GROUPED_GEMM | P, F=3008) == SHAPE


def test_mlp_workspace_covers_both_algorithms(L):
    T, D, F, E, k = 8192, 2880, 2880, 32, 4
    P = T * k
    n = L.moe_expert_mlp_workspace_size(T, D, F, E, k)
    y = 4 * P * D
    assert n >= y + 2 * P * F                      # streaming: y + fp16 h
    # grouped GEMM: y + fp16 h + x as 2 fp8 terms (144 bytes per 64 elements)
    assert n >= y + 2 * P * F + T * (D // 64) * 144


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        moe.mxfp4_quantize(torch.zeros(4, 64, dtype=torch.bfloat16))
