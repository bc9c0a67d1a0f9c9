"""Build step for the HIP library (hipcc, gfx950)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
# the step kernels, state codec and core ABI; the activation codec
SOURCES = [os.path.join(CSRC, "coat_fp8.hip"), os.path.join(CSRC, "act_fp8.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcoat_fp8.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # explicit fma only: the fp64 moment chain must not be re-associated
    "-ffp-contract=off",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    """Compile the csrc/*.hip sources into libcoat_fp8.so next to this file."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I" + INCLUDE, "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(res.stderr)
    os.replace(tmp, LIB)
    return LIB


def build_ceiling_probe() -> str:
    """Compile bench_ceiling.hip (the memory-pattern instrument of bench.py
    --ceiling, not part of the library) into libbench_ceiling.so at the root."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = os.path.join(ROOT, "libbench_ceiling.so")
    flags = [f for f in HIPCC_FLAGS if f != "-ffp-contract=off"]
    res = subprocess.run([hipcc, *flags, "-o", out + ".tmp", os.path.join(ROOT, "bench_ceiling.hip")],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
