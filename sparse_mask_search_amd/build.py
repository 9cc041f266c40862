"""Build libtsenor.so (HIP, gfx950) in-tree with hipcc.

    python -m sparse_mask_search_amd.build

Every HIP source is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtsenor.so")
SOURCES = ["tsenor_abi.cpp", "tsenor_kernels.hip", "tsenor_spmm.hip", "tsenor_bench.hip"]
ARCH = os.environ.get("TSENOR_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + _flags() + ["-fPIC", "-shared", "-o", tmp]
    cmd += ["-x", "hip"] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def device_asm(source: str, out: str) -> str:
    """gfx950 assembly of one HIP source, compiled as for the library."""
    cmd = [hipcc()] + _flags() + ["--cuda-device-only", "-S", "-o", out,
                                  os.path.join(CSRC, source)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
