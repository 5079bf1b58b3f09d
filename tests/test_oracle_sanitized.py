"""The CPU oracle under the address and undefined-behaviour sanitizers:
seeded random round trips (own and foreign codebooks, all chunk-size
classes) and decodes of damaged payloads and metadata, which must end in a
status code and never in an access outside the buffers."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_fuzz"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-static-libasan", "-static-libubsan",
           "-Wall", "-Wextra", "-Werror",
           os.path.join(ROOT, "oracle", "splitzip_oracle.c"),
           os.path.join(ROOT, "tests", "c_smoke", "oracle_fuzz.c"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe), "600"], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "0 round-trip failures" in run.stdout
