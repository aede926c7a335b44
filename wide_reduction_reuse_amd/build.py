"""Build libcredit.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m wide_reduction_reuse_amd.build [--jobs N]

Objects go to ``wide_reduction_reuse_amd/_build/``; the library is written to
``wide_reduction_reuse_amd/libcredit.so``.  Every call recompiles.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcredit.so")
INCLUDE = os.path.join(ROOT, "include")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU ops are disabled for all device code; the host pass warns
# that it does not know the feature, which is harmless.
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument",
          "-I", INCLUDE, "-I", CSRC]

SOURCES = ["inst_softmax.hip", "inst_layernorm.hip", "inst_rmsnorm.hip", "inst_softmax_bwd.hip",
           "inst_layernorm_bwd.hip", "inst_quantize.hip", "inst_misc.hip", "noalloc.hip", "api.cpp", "planner.cpp"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), out))
    return obj


def build(jobs: int = 0, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    # -z defs: every symbol the library uses must resolve at link time (a
    # missing translation unit fails here, not at load time)
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-Wl,-z,defs", "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    a = ap.parse_args(argv)
    build(a.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
