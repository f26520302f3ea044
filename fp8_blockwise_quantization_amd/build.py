"""Build the gfx950 HIP library ``libfp8rl.so`` in-tree with hipcc.

Usage: ``python -m fp8_blockwise_quantization_amd.build`` (or call ``build()``).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libfp8rl.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ("quant.hip", "tensor_quant.hip", "transpose_quant.hip", "gemm.hip", "fp8rl_abi.hip")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed FP32 instructions.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc_path() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libfp8rl")


def build(verbose: bool = False, extra_flags=(), out_path: str | None = None) -> str:
    """Compile every HIP source into ``libfp8rl.so`` next to this file (or into ``out_path``);
    returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    out = out_path or LIB_PATH
    tmp = out + ".tmp"
    cmd = [hipcc_path(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
           "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
