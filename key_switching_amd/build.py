"""Build libpc.so (the gfx950 key-switching library) in place with hipcc.

Usage: python -m key_switching_amd.build   (or key_switching_amd.build.build())
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/kernels.hip", "csrc/capi.hip"]
# kernels.hip is compiled once per launcher group (-DPC_PART=n), in parallel
KERNEL_PARTS = 5
OBJ_DIR = os.path.join(HERE, "_build")
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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source into key_switching_amd/libpc.so; returns its path.

    kernels.hip is compiled as KERNEL_PARTS objects (one launcher group each)
    and capi.hip as one, in parallel, then linked into the shared library."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    comp = [f for f in HIPCC_FLAGS if f != "-shared"]
    kern = os.path.join(HERE, SOURCES[0])
    units = [([f"-DPC_PART={i}"], kern, os.path.join(OBJ_DIR, f"kernels_p{i}.o"))
             for i in range(1, KERNEL_PARTS + 1)]
    units.append(([], os.path.join(HERE, SOURCES[1]), os.path.join(OBJ_DIR, "capi.o")))
    cmds = [[hipcc(), *comp, *defs, *inc, "-c", src, "-o", obj] for defs, src, obj in units]
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1), 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *[obj for _, _, obj in units], "-o", tmp], verbose)
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
