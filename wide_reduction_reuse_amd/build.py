"""Build libcredit.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m wide_reduction_reuse_amd.build [--jobs N] [--asan]

Objects go to ``wide_reduction_reuse_amd/_build/``; the library is written to
``wide_reduction_reuse_amd/libcredit.so``.  Every call recompiles.  --asan
also builds ``_build/libcredit_asan.so``, the same library with its host code
instrumented by AddressSanitizer, for the CPU tests of the host code.
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
           "inst_layernorm_bwd.hip", "inst_quantize.hip", "inst_misc.hip", "noalloc.hip", "lnbwd_params.hip", "api.cpp",
           "planner.cpp"]


# Host-side AddressSanitizer variant (libcredit_asan.so, for the CPU tests of
# the host code): the host pass is instrumented, device code is unchanged.
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
ASAN_BUILD = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(BUILD, "libcredit_asan.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime a process must preload to load
    libcredit_asan.so (the interpreter itself is not instrumented)."""
    out = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                         stderr=subprocess.DEVNULL, text=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        import glob
        found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        out = found[0] if found else ""
    return out


def _compile(src: str, asan: bool = False) -> str:
    outdir = ASAN_BUILD if asan else BUILD
    obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + (ASAN_FLAGS if asan else []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), out))
    return obj


def build(jobs: int = 0, verbose: bool = False, asan: bool = False) -> str:
    """Compile every source and link the library; asan=True builds the
    host-ASan variant instead (ASAN_LIB)."""
    os.makedirs(ASAN_BUILD if asan else BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, asan), SOURCES))
    lib = ASAN_LIB if asan else LIB
    tmp = lib + ".tmp%d" % os.getpid()
    # -z defs: every symbol the library uses must resolve at link time (a
    # missing translation unit fails here, not at load time); the ASan
    # variant leaves the sanitizer's symbols to the preloaded runtime
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + ([] if asan else ["-Wl,-z,defs"]) + ["-o", tmp]
    subprocess.check_call(cmd + objs)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--asan", action="store_true", help="also build the host-ASan variant")
    a = ap.parse_args(argv)
    build(a.jobs, verbose=True)
    if a.asan:
        build(a.jobs, verbose=True, asan=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
