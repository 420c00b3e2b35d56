"""Host-side sanitizer runs (no GPU): the CPU oracle and the C ABI's argument validation and
split planner, each built with gcc/g++ -fsanitize=address,undefined and driven by a small
C/C++ program (tests/host/oracle_sanitize.c, tests/host/abi_host.cpp; the ABI build replaces
the kernel launchers with counting stubs). A sanitizer finding aborts the driver."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd_build, exe):
    subprocess.run(cmd_build, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    out = _run(["gcc", "-std=c11", *SAN, "-fno-fast-math", "-ffp-contract=off", "-pthread",
                os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), os.path.join(HERE, "host", "oracle_sanitize.c"),
                "-lm", "-o", exe], exe)
    assert "0 non-finite" in out


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    out = _run(["g++", "-std=c++17", *SAN, "-DNVFP4_HOST_ABI_TEST", "-I", os.path.join(HERE, "host"),
                "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "quantized_kv_decode_amd", "csrc"),
                os.path.join(ROOT, "quantized_kv_decode_amd", "csrc", "api.cpp"),
                os.path.join(HERE, "host", "abi_host.cpp"), "-o", exe], exe)
    assert "0 failures" in out
