"""Build the HIP library paged_kv_cache_gca_amd/libgca.so for gfx950 (hipcc)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(_HERE, "csrc")
LIB = os.path.join(_HERE, "libgca.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gca_runtime.hip", "gca_kernels.hip", "gca_plan.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # per-thread arrays stay in registers: the kernels budget LDS themselves
    # (two attention workgroups per CU), so no private array is moved there
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
