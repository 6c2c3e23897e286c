"""Builds libflash_attn.so in this package directory with hipcc for gfx950.

    python -m exact_io_aware_flash_amd.build [--verbose]

The library is compiled in-tree so that it travels with the source tree; nothing is installed.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["api.cpp", "fwd_bf16.hip", "fwd_fp8.hip", "bwd_bf16.hip", "f32.hip", "noalloc.hip"]
HEADERS = ["fa_common.h", "fa_kernels.h"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libflash_attn.so")


# Checking builds of the same sources, loaded by tests through FLASH_ATTN_LIB:
#  check: every asynchronous copy into LDS first fills its destination with NaN (-DFA_CHECK), so a
#         read that runs ahead of its copy shows up in the results;
#  asan:  host code (the argument validation of the C ABI) built with AddressSanitizer and
#         UndefinedBehaviorSanitizer; the device code is built as usual.
VARIANTS = {
    "main": ("libflash_attn.so", []),
    "check": ("libflash_attn_check.so", ["-DFA_CHECK"]),
    "asan": ("libflash_attn_asan.so", ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                                       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
                                       "-fno-omit-frame-pointer"]),
}


def variant_path(name: str) -> str:
    return os.path.join(PKG, VARIANTS[name][0])


def build(verbose: bool = False, extra_flags: list[str] | None = None, variant: str = "main") -> str:
    out = variant_path(variant)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *VARIANTS[variant][1], *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
           "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is expected
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}) for the {variant} build:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list[str]:
    """The library and its checking builds, compiled side by side."""
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(len(VARIANTS)) as ex:
        return list(ex.map(lambda v: build(verbose, variant=v), VARIANTS))


def sanitizer_runtime() -> str | None:
    """The compiler's AddressSanitizer runtime (preloaded into a process that loads the asan build)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    import glob

    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


if __name__ == "__main__":
    for p in build_all(verbose="--verbose" in sys.argv):
        print(p)
