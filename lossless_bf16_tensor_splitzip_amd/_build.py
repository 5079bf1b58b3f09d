"""Build of the HIP libraries (gfx950 only): ``_lib/libsplitzip.so``, the
codec, and ``_lib/libsplitzip_ceiling.so``, the reference memory streams its
kernels are measured against."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "splitzip.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libsplitzip.so")
CEILING_SRC = os.path.join(PKG, "csrc", "ceiling.hip")
CEILING_LIB_PATH = os.path.join(LIB_DIR, "libsplitzip_ceiling.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str, lib_path: str, verbose: bool) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = lib_path + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, src, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose: bool = False) -> str:
    """Compile both libraries (always recompiles); returns the codec's path."""
    _compile(CEILING_SRC, CEILING_LIB_PATH, verbose)
    return _compile(SRC, LIB_PATH, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
