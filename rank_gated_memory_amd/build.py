"""Build libgsi.so in-tree for gfx950 with hipcc (no JIT, no cache)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "gsi_api.cpp"), os.path.join(PKG, "csrc", "gsi_kernels.hip"),
           os.path.join(PKG, "csrc", "gsi_batched.hip"), os.path.join(PKG, "csrc", "gsi_calib.hip"),
           os.path.join(PKG, "csrc", "gsi_noalloc.hip")]
OUT = os.path.join(PKG, "libgsi.so")

COMMON = [
    "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
FLAGS = ["-O3", *COMMON]
# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (each
# -fsanitize= applies to the host pass only; device code is built as usual),
# warnings as errors.  Loaded through GSI_LIBRARY with the ASan runtime
# preloaded, for the CPU-side tests of argument checking and plan building.
SAN_FLAGS = ["-O1", "-g", "-Werror", *COMMON,
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_OUT = os.path.join(ROOT, "_build", "libgsi_hostsan.so")
# The per-job trace of the single-launch stack (instrumented, slower): loaded
# through GSI_LIBRARY by `bench.py --trace`; exports gsi_trace_read/_reset.
TRACE_FLAGS = [*FLAGS, "-DGSI_TRACE=1"]
TRACE_OUT = os.path.join(PKG, "libgsi_trace.so")


def _compile(flags, out, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [hipcc, *flags, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    return _compile(FLAGS, OUT, verbose)


def build_traced(verbose: bool = False) -> str:
    """The instrumented build (TRACE_FLAGS) at TRACE_OUT."""
    return _compile(TRACE_FLAGS, TRACE_OUT, verbose)


def build_sanitized(verbose: bool = False) -> str:
    """The host-sanitizer build (SAN_FLAGS) at SAN_OUT."""
    return _compile(SAN_FLAGS, SAN_OUT, verbose)


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (to preload into Python)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return hits[-1]


if __name__ == "__main__":
    print(build(verbose=True))
