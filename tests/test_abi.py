"""The C ABI library loads, exports every symbol the header declares, and
rejects bad arguments before enqueuing anything (no GPU needed: every call
here fails validation on the host, or -- on a host without a gfx950 -- the
device check that follows it)."""

import ctypes
import os
import re

import pytest

import mxfp4_quantized_mixture_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")

OK, NULL, SHAPE, WS, ENUM, HIP, DEVICE, ALIGN = range(8)


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
            "moe_abi_version", "moe_expert_mlp_bf16", "moe_expert_mlp_bf16_ex",
            "moe_expert_mlp_bf16_workspace_size", "moe_layer_decode", "moe_layer_decode_ex",
            "moe_layer_decode_init", "moe_layer_decode_error",
            "moe_layer_decode_workspace_size"} <= names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_no_internal_symbols_exported():
    out = os.popen("nm -D --defined-only %s" % moe.LIB_PATH).read()
    text_syms = [l.split()[-1] for l in out.splitlines() if " T " in l]
    assert set(text_syms) == set(declared_functions())


def test_probe_library_exports_its_header():
    from mxfp4_quantized_mixture_amd import build as B
    text = open(os.path.join(ROOT, "include", "moe_probe.h")).read()
    declared = set(re.findall(r"MOE_PROBE_API\s+[\w\s\*]+?\b(\w+)\s*\(", text))
    assert declared == {"moe_probe_read", "moe_probe_read_grouped", "moe_probe_mfma",
                        "moe_probe_mfma_flops"}
    out = os.popen("nm -D --defined-only %s" % B.PROBE_LIB).read()
    assert {l.split()[-1] for l in out.splitlines() if " T " in l} == declared
    P = ctypes.CDLL(B.PROBE_LIB)
    P.moe_probe_mfma_flops.restype = ctypes.c_double
    assert P.moe_probe_mfma_flops(1) == 2 * 32 * 32 * 64
    assert P.moe_probe_mfma_flops(4) == 2 * 32 * 32 * 16
    assert P.moe_probe_mfma_flops(9) == 0
    P.moe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
    assert P.moe_probe_read(None, 1 << 20, 8, FAKE, None) == 1        # bad arguments
    assert P.moe_probe_read(FAKE + 4, 1 << 20, 8, FAKE, None) == 1    # misaligned
    assert P.moe_probe_mfma(9, 8, 1, FAKE, None) == 4                 # unknown kind
    P.moe_probe_read_grouped.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert P.moe_probe_read_grouped(None, 4, 8, 1, FAKE, None) == 1      # bad arguments
    assert P.moe_probe_read_grouped(FAKE + 4, 4, 8, 1, FAKE, None) == 1  # misaligned
    assert P.moe_probe_read_grouped(FAKE, 4, 8, 3, FAKE, None) == 1      # 3 does not divide 64
    assert P.moe_probe_read_grouped(FAKE, 0, 8, 1, FAKE, None) == 1      # no chunks


def test_status_strings(L):
    assert L.moe_status_string(OK) == b"ok"
    names = set()
    for s in range(1, 8):
        assert L.moe_status_string(s) and L.moe_status_string(s) != b"ok"
        names.add(L.moe_status_string(s))
    assert len(names) == 7
    assert b"gfx950" in L.moe_status_string(DEVICE)
    assert L.moe_status_string(99) == b"unknown status"
    assert L.moe_abi_version() == 4 == moe.ABI_VERSION


def test_header_status_codes_match():
    text = open(HEADER).read()
    for name, code in (("MOE_OK", OK), ("MOE_ERR_NULL", NULL), ("MOE_ERR_SHAPE", SHAPE),
                       ("MOE_ERR_WORKSPACE", WS), ("MOE_ERR_ENUM", ENUM), ("MOE_ERR_HIP", HIP),
                       ("MOE_ERR_DEVICE", DEVICE), ("MOE_ERR_ALIGN", ALIGN)):
        assert re.search(r"\b%s = %d\b" % (name, code), text), name


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
    # mxfp4_quantize(w, rows, K, q, s, scale_rule, stream)
    assert L.mxfp4_quantize(FAKE, 4, 48, FAKE, FAKE, 0, None) == SHAPE
    assert L.mxfp4_quantize(FAKE, -1, 64, FAKE, FAKE, 0, None) == SHAPE
    assert L.mxfp4_quantize(FAKE, 4, 64, FAKE, FAKE, 3, None) == ENUM
    # mxfp4_quantize_ex(w, rows, K, q, s, scale_rule, rounding, seed, stream)
    assert L.mxfp4_quantize_ex(FAKE, 4, 64, FAKE, FAKE, 2, 2, 0, None) == ENUM   # rounding
    assert L.mxfp4_quantize_ex(FAKE, 4, 64, FAKE, FAKE, 3, 1, 0, None) == ENUM   # rule
    assert L.mxfp4_quantize_ex(FAKE, 4, 48, FAKE, FAKE, 2, 1, 0, None) == SHAPE
    assert L.mxfp4_quantize_ex(None, 4, 64, FAKE, FAKE, 2, 1, 0, None) == NULL
    assert L.mxfp4_quantize_ex(None, 0, 64, None, None, 2, 1, 0, None) == OK
    assert L.mxfp4_quantize(None, 4, 64, FAKE, FAKE, 0, None) == NULL
    assert L.mxfp4_quantize(FAKE + 2, 4, 64, FAKE, FAKE, 0, None) == ALIGN
    assert L.mxfp4_quantize(None, 0, 64, None, None, 0, None) == OK    # empty: nothing to do
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
                            out, FAKE, ws_bytes, None)


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
    assert _mlp_ex(L, moe.MLP_GROUPED_GEMM, F=8256) == SHAPE    # contraction limit
    assert _mlp_ex(L, moe.MLP_GROUPED_GEMM, D=8256) == SHAPE
    assert _mlp_ex(L, moe.MLP_STREAM, F=3008) == SHAPE          # streaming kernels' LDS budget
    assert _mlp_ex(L, moe.MLP_STREAM, D=3904) == SHAPE
    assert _mlp_ex(L, moe.MLP_AUTO, D=4000) == SHAPE            # neither algorithm takes it
    assert _mlp_ex(L, moe.MLP_STREAM, F=3008, out=None) == NULL # pointers are checked first
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
    assert n >= y + 4 * P * F                      # streaming: y + fp32 h
    # grouped GEMM: y + h as fp6 term rows + x as fp6 term rows (160 bytes
    # per 64 elements each)
    assert n >= y + P * (F // 64) * 160 + T * (D // 64) * 160


def _bf16(L, T=8, D=64, F=64, E=4, k=2, out=FAKE, ws_bytes=None, w13=FAKE, events=None):
    if ws_bytes is None:
        ws_bytes = L.moe_expert_mlp_bf16_workspace_size(T, D, F, E, k) or 1 << 20
    return L.moe_expert_mlp_bf16_ex(FAKE, w13, FAKE, FAKE, FAKE, FAKE, FAKE, T, D, F, E, k, out,
                                    FAKE, ws_bytes, events, None)


def test_bf16_mlp_workspace_and_validation(L):
    T, D, F, E, k = 32, 2880, 2880, 32, 4
    assert L.moe_expert_mlp_bf16_workspace_size(T, D, F, E, k) >= 4 * T * k * (D + F)
    assert L.moe_expert_mlp_bf16_workspace_size(8, 64, 48, 4, 2) == 0   # F % 32
    assert L.moe_expert_mlp_bf16_workspace_size(0, 64, 64, 4, 2) == 0   # T < 1
    assert _bf16(L, F=40) == SHAPE
    assert _bf16(L, D=48) == SHAPE
    assert _bf16(L, k=5, E=4) == SHAPE
    assert _bf16(L, out=None) == NULL
    assert _bf16(L, w13=None) == NULL
    assert _bf16(L, ws_bytes=100) == WS
    assert _bf16(L, w13=FAKE + 4) == ALIGN
    assert L.moe_expert_mlp_bf16(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 64, 40, 4, 2,
                                 FAKE, FAKE, 1 << 20, None) == SHAPE


def _decode(L, T=8, D=64, F=64, E=4, k=2, out=FAKE, ws_bytes=None, flags=0, spin=1000,
            x=FAKE):
    if ws_bytes is None:
        ws_bytes = L.moe_layer_decode_workspace_size(T, D, F, E, k) or 1 << 20
    return L.moe_layer_decode_ex(x, FAKE, None, FAKE, FAKE, FAKE, FAKE, T, D, F, E, k, FAKE,
                                 FAKE, FAKE, FAKE, FAKE, FAKE, out, FAKE, ws_bytes, flags, spin,
                                 None, None)


def test_decode_workspace_and_validation(L):
    T, D, F, E, k = 32, 2880, 2880, 32, 4
    n = L.moe_layer_decode_workspace_size(T, D, F, E, k)
    assert n >= 256 + 4 * T * k * (D + F)                     # control block, y, fp32 h
    assert L.moe_layer_decode_workspace_size(65, 64, 64, 4, 2) == 0      # T > 64
    assert L.moe_layer_decode_workspace_size(64, 64, 64, 256, 2) == 0    # T E > 8192
    assert L.moe_layer_decode_workspace_size(8, 64, 48, 4, 2) == 0       # F % 32
    assert L.moe_layer_decode_workspace_size(8, 64, 4160, 4, 2) == 0     # streaming LDS budget
    assert _decode(L, flags=3) == ENUM
    assert _decode(L, flags=moe.MLP_STREAM) == ENUM                      # only the packed flag
    assert _decode(L, T=65) == SHAPE
    assert _decode(L, F=40) == SHAPE
    assert _decode(L, spin=-1) == SHAPE
    assert _decode(L, D=96, flags=moe.MLP_WEIGHTS_PACKED) == SHAPE       # packed needs D % 64
    assert _decode(L, out=None) == NULL
    assert _decode(L, x=None) == NULL
    assert _decode(L, ws_bytes=100) == WS
    assert _decode(L, x=FAKE + 8) == ALIGN
    assert L.moe_layer_decode_init(None, 1024, None) == NULL
    assert L.moe_layer_decode_init(FAKE, 16, None) == WS
    assert L.moe_layer_decode_error(FAKE, None, None) == NULL


def _gpu_present():
    import torch
    return torch.cuda.is_available()


# On a host without a gfx950 every call that passes validation stops at the
# device check, before anything is enqueued (these calls would launch kernels
# on fake pointers on a GPU host, so they run only where there is none).
@pytest.mark.skipif(_gpu_present(), reason="needs a host without a GPU")
def test_valid_calls_without_a_gfx950_return_device_error(L):
    assert L.mxfp4_quantize(FAKE, 4, 64, FAKE, FAKE, 0, None) == DEVICE
    assert L.mxfp4_quantize_ex(FAKE, 4, 64, FAKE, FAKE, 2, 1, 7, None) == DEVICE
    assert L.mxfp4_dequantize(FAKE, FAKE, 4, 64, FAKE, None) == DEVICE
    assert L.mxfp4_pack(FAKE, 32, 64, FAKE + 4096, None) == DEVICE
    assert _route(L) == DEVICE
    assert _mlp(L) == DEVICE
    assert _mlp_ex(L, moe.MLP_GROUPED_GEMM) == DEVICE
    assert _mlp_ex(L, moe.MLP_AUTO, D=3904) == DEVICE           # taken by the grouped GEMM
    assert _bf16(L) == DEVICE
    assert _decode(L) == DEVICE
    assert L.moe_layer_decode_init(FAKE, 1024, None) == DEVICE
    # argument errors still win over the device check
    assert _mlp(L, F=40) == SHAPE
    assert _bf16(L, F=40) == SHAPE


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        moe.mxfp4_quantize(torch.zeros(4, 64, dtype=torch.bfloat16))
