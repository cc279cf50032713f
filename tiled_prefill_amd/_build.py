"""Build libattn.so (HIP kernels + C-ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")

SOURCES = ["attn_fwd.hip", "attn_fwd_f32.hip", "attn_decode.hip", "attn_prefill.hip", "attn_mla.hip", "attn_bwd.hip",
           "attn_scratch.hip", "attn_tools.hip", "attn_api.cpp"]
HEADERS = ["attn_plan.h", "attn_kernels.h", "attn_device.h"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 VALU forms are kept out of every code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source into tiled_prefill_amd/libattn.so (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags or []) + [
        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp,
    ] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# library (planner, C-ABI and launch code instrumented; the device code is
# built as usual). Loaded in place of libattn.so through ATTN_LIB, with the
# sanitizer runtime preloaded (asan_runtime()), by the CPU test suite.
SANITIZE_FLAGS = [
    "-Xarch_host", "-g",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
]


def build_sanitized(out_dir: str, verbose: bool = False) -> str:
    out = os.path.join(out_dir, "libattn_asan.so")
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O2"] + SANITIZE_FLAGS
    cmd = [hipcc()] + flags + ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", out] + [
        os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    return out


def asan_runtime() -> str:
    """The compiler's shared ASan runtime (it carries the UBSan handlers too)."""
    return subprocess.check_output([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
