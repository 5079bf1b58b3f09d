"""Build of the plain-C driver of the C ABI (tests/c_smoke/_build/)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "splitzip_c_smoke.c")
EXE = os.path.join(HERE, "_build", "splitzip_c_smoke")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror",
           # the HIP runtime API header serves several platforms; this names ours
           "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
           SRC, "-o", EXE,
           "-L", os.path.join(ROOT, "lossless_bf16_tensor_splitzip_amd", "_lib"), "-lsplitzip",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../../lossless_bf16_tensor_splitzip_amd/_lib",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the C driver failed:\n" + res.stdout + res.stderr)
    return EXE


if __name__ == "__main__":
    print(build())
