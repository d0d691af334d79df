"""Build libmoe_mxfp4.so (the layer) and libmoe_probe.so (achievable-peak
microbenchmarks) in-tree with hipcc for gfx950.

    python -m mxfp4_quantized_mixture_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_mxfp4.so")
SOURCES = ["quantize.hip", "route.hip", "expert_mlp.hip", "expert_gemm.hip", "expert_bf16.hip",
           "decode.hip", "api.hip"]
PROBE_LIB = os.path.join(PKG, "libmoe_probe.so")
PROBE_SOURCES = ["probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
    # no packed fp32 (v_pk_*_f32) instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(sources, out, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source: libmoe_mxfp4.so and libmoe_probe.so (always
    recompiles).  Returns the layer library's path."""
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
