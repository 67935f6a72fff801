"""Build libpc.so (the gfx950 key-switching library) in place with hipcc.

Usage: python -m key_switching_amd.build   (or key_switching_amd.build.build())
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/kernels.hip", "csrc/capi.hip"]
LIB = os.path.join(HERE, "libpc.so")
PROBE_SRC = os.path.join(HERE, "rate_probe.hip")
PROBE = os.path.join(HERE, "rate_probe")  # instruction-rate probe (measurement tool, not part of the library)

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=gfx950",
    # keep the compiler from forming packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every HIP source into key_switching_amd/libpc.so; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(HERE, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


def build_probe(verbose: bool = False) -> str:
    """Compile the instruction-rate probe (key_switching_amd/rate_probe)."""
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [hipcc(), *flags, PROBE_SRC, "-o", PROBE]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}")
    return PROBE


if __name__ == "__main__":
    build(verbose=True)
    build_probe(verbose=True)
    print("built", LIB, "and", PROBE, file=sys.stderr)
