"""Build the gfx950 HIP library in-tree: fp8_gemm_amd/libfp8gemm.so."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "fp8_gemm.hip")
DEPS = [os.path.join(HERE, "csrc", f) for f in ("kernels.hpp", "device_common.hpp")] + \
       [os.path.join(ROOT, "include", "fp8_gemm.h")]
LIB = os.path.join(HERE, "libfp8gemm.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed FP32 VALU ops (v_pk_add/mul/fma_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(force: bool = True) -> str:
    """Compile the library.  Always recompiles when force is True."""
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in [SRC] + DEPS)
        if os.path.getmtime(LIB) >= newest:
            return LIB
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + [SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
