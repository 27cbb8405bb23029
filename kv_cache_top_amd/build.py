"""Build libpariskv.so (HIP for gfx950) in-tree.

    python -m kv_cache_top_amd.build [--verbose] [--sanitize]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpariskv.so")

SOURCES = ["pk_api.hip", "pk_tables.cpp"]
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # fp32 operations that decide integer codes follow a fixed order: no fusing
    "-ffp-contract=off",
    # no packed fp32 arithmetic in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpariskv.so)")


# host code only: AddressSanitizer and UndefinedBehaviorSanitizer on the
# runtime's C++ (argument checks, tables, launch plans); device code is built
# as usual.  Load the result with PARISKV_LIB and the sanitizer runtime
# preloaded (see sanitizer_runtime()).
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
LIB_SANITIZED = os.path.join(PKG, "libpariskv_hostsan.so")


def sanitizer_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime (to LD_PRELOAD into python)."""
    out = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return out.stdout.strip()


def build(verbose: bool = False, extra: list[str] | None = None, sanitize: bool = False) -> str:
    """Compile every source into kv_cache_top_amd/libpariskv.so (with sanitize:
    libpariskv_hostsan.so, host code sanitized); returns its path."""
    out_lib = LIB_SANITIZED if sanitize else LIB
    tmp = out_lib + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(SANITIZE_FLAGS if sanitize else []), *(extra or []), "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs))
    os.replace(tmp, out_lib)
    return out_lib


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, sanitize="--sanitize" in sys.argv))
