"""Build libfavor.so in-tree for gfx950 (MI355X).

    python random_feature_amd/build.py [--jobs N] [--verbose] [--tools]

(Run it as a script: importing the package itself needs the built library.)

Each HIP source is compiled separately (in parallel) with hipcc for
--offload-arch=gfx950; the host-side Omega generator is compiled with g++
without floating-point contraction or fast-math (its fp64 arithmetic must
round exactly as written). Objects go to random_feature_amd/_build/, the
shared library to random_feature_amd/libfavor.so. --tools also builds the
pipe-rate microbenchmark (random_feature_amd/tools/rates.hip) as
random_feature_amd/_build/rates; it is measurement tooling, not part of the library.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfavor.so")
ARCH = "gfx950"

HIP_SOURCES = ["favor_bidir.hip", "favor_causal.hip", "favor_decode.hip", "favor_backward.hip",
               "favor_causal_bwd.hip"]
HOST_HIP_SOURCES = ["favor_api.cpp", "favor_timing.cpp"]       # host code that calls the HIP runtime
PLAIN_SOURCES = ["omega_host.cpp"]         # pure C++ (no HIP)

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfavor)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(jobs: int | None = None, verbose: bool = False, tools: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([hipcc, "-O2", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"),
                     "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in PLAIN_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", "-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
                     "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    n = jobs or min(len(cmds), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=n) as ex:
        for out in ex.map(lambda c: _run(c, verbose), cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    if tools:
        build_tools(verbose)
    return LIB


def build_tools(verbose: bool = False) -> str:
    """The pipe-rate microbenchmark (exp, FMA and MFMA issue rates on the device), a standalone program."""
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "rates")
    _run([_hipcc(), *[f for f in HIPCC_FLAGS if f != "-fPIC"],
          os.path.join(ROOT, "random_feature_amd", "tools", "rates.hip"), "-o", exe], verbose)
    return exe


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--tools", action="store_true", help="also build the pipe-rate microbenchmark")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose, a.tools))


if __name__ == "__main__":
    sys.exit(main())
