"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU.

Every source of libsgdstep is compiled with the sanitizers on its host side
only (device code is built as usual and never launched), linked with
tests/native/host_check.cpp, and run: the planner for the benchmark networks
and a ragged one, every query entry point, the workspace computations and
the argument checks of the compute entry points.  Any out-of-bounds access,
overflow or undefined operation in that host code aborts the run.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(shutil.which("hipcc") is None or not os.path.exists(CLANG), reason="needs hipcc")
def test_library_host_code_clean_under_asan_and_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include")]
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]

    def compile_hip(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = ["hipcc", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, *inc, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    srcs = sorted(glob.glob(os.path.join(ROOT, "sgd_cnns_amd", "csrc", "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(6, len(srcs))) as ex:
        objs = list(ex.map(compile_hip, srcs))
    drv = str(tmp_path / "host_check.o")
    subprocess.run([CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *SAN, *inc, "-c",
                    os.path.join(ROOT, "tests", "native", "host_check.cpp"), "-o", drv], check=True)
    exe = str(tmp_path / "host_check")
    subprocess.run([CLANG, *SAN, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "ok" in r.stdout
