"""Build librf.so in-tree with hipcc for gfx950.

    python -m cascaded_reductions_amd.build [-v]

Every HIP/C++ source under csrc/ is compiled (in parallel) into _build/ and
linked into cascaded_reductions_amd/librf.so, replacing it atomically.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librf.so")

ARCH = "gfx950"
CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # Packed fp32 VALU forms are disabled: the compiler emits ordinary scalar fp32 ops instead.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Kernel arguments preloaded into SGPRs at dispatch (gfx950), so a wave starts without
    # waiting for a scalar load of its arguments: 1-7% off the launch-bound steps.
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines()
                    if "packed-fp32-ops" not in ln and "not a recognized feature" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link librf.so. Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_run, [hipcc, *CXXFLAGS, "-x", "hip", "-c", s, "-o", o], verbose)
                for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = LIB + f".tmp{os.getpid()}"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
