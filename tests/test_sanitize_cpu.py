"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): the two fp64 oracles, and the C ABI's validation and buffer layout
with the kernel launchers replaced by recording stubs.  Each driver exits
non-zero on a failed check, and a sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return res.returncode, res.stdout + res.stderr


def _check(exe):
    rc, out = _run([exe], env=ENV, timeout=600)
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert rc == 0, out[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracles_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-std=c11", "-pthread", *SAN, "-o", exe,
                    os.path.join(HERE, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "wkv7_oracle.c"),
                    os.path.join(ROOT, "oracle", "rwkv8_oracle.c"), "-lm"])
    assert rc == 0, out
    _check(exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_abi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "linear_attention_rnn_wkv7_amd", "csrc")
    rc, out = _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc, "-o", exe,
                    os.path.join(HERE, "abi_driver.cpp"), os.path.join(csrc, "wkv7_abi.cpp")])
    assert rc == 0, out
    _check(exe)
