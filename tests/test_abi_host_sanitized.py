"""The host side of the C ABI (sizes, status strings, argument checks) under
AddressSanitizer/UBSan: the library is rebuilt with the host sanitizers
(device code unchanged) and driven from a small C program without a GPU."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs ROCm")
def test_abi_host_under_sanitizers(tmp_path):
    lib = tmp_path / "libsplitzip_san.so"
    build = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # sanitizers for the host code only
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"),
             os.path.join(ROOT, "lossless_bf16_tensor_splitzip_amd", "csrc", "splitzip.hip"),
             "-o", str(lib)]
    res = subprocess.run(build, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    exe = tmp_path / "abi_host_check"
    drv = [CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_smoke", "abi_host_check.c"), "-o", str(exe),
           "-L", str(tmp_path), "-lsplitzip_san", "-Wl,-rpath," + str(tmp_path)]
    res = subprocess.run(drv, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "0 failures" in run.stdout
