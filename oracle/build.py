"""Compile the CPU oracle into oracle/libgca_oracle.so (plain g++, no HIP)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "gca_oracle.cpp")
    out = os.path.join(_HERE, "libgca_oracle.so")
    tmp = out + ".tmp"
    # x86-64-v3 (AVX2) so the library also runs on the GPU hosts' CPUs
    cmd = ["g++", "-std=c++17", "-O3", "-march=x86-64-v3", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-pthread", src, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
