"""Build libbsa.so, the HIP library behind the C ABI in include/bsa.h, for gfx950.

Run ``python -m long_context_attention_sparse_amd.build`` (or call ``build()``).
The library lands next to this file, where the binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbsa.so")
# translation units and their extra flags
SOURCES = [
    ("bsa_api.hip", []),
    ("kernels_stream.hip", []),
    ("kernels_check.hip", []),
    # the tile kernels never create NaNs (masked scores are -inf, handled explicitly), so
    # max needs no NaN-quieting canonicalisation: plain v_max/v_max3 in the softmax
    ("kernels_tile.hip", ["-fno-honor-nans", "-mno-amdgpu-ieee"]),
    ("kernels_select.hip", ["-fno-honor-nans", "-mno-amdgpu-ieee"]),
    ("kernels_bwd.hip", ["-fno-honor-nans", "-mno-amdgpu-ieee"]),
]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the C ABI layer (argument
# validation, plans, launch set-up); the device code is built as usual.  The sanitizer runtime is
# not linked into the library: a process loading it preloads libclang_rt.asan (sanitizer_runtime()).
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(PKG, "libbsa_sanitized.so")


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime of the ROCm compiler (for LD_PRELOAD)."""
    res = subprocess.run([os.path.join(os.path.dirname(hipcc()), "amdclang++"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def build(verbose: bool = False, extra_flags=None, sanitize: bool = False) -> str:
    """Compile every HIP translation unit and link libbsa.so (always recompiles).  With
    sanitize=True the C ABI layer (bsa_api.hip) is built with host ASan/UBSan into
    libbsa_sanitized.so instead, beside the regular library, which is left alone."""
    objdir = os.path.join(PKG, "_build_sanitized" if sanitize else "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src, flags in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        san = SANITIZE_FLAGS if sanitize and src == "bsa_api.hip" else []
        _run([hipcc(), *HIP_FLAGS, *flags, *san, *(extra_flags or []), "-I", os.path.join(ROOT, "include"), "-I",
              CSRC, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
