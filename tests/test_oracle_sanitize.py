"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/sanitize_check.c drives every oracle function on small ragged shapes
with exactly sized heap buffers; built with -fsanitize=address,undefined and
-fno-sanitize-recover=all, any out-of-bounds access, overflow or undefined
operation aborts the run.  Host code only: nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-ffp-contract=off", "-Wno-unknown-pragmas",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "oracle", "sanitize_check.c"),
           "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert "ok" in r.stdout
