"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU code: the
oracle (oracle/kq_oracle.c) and the library's host helpers
(csrc/kq_host.cpp), each linked into a driver under tests/sanitize/ that
calls every entry point on exactly sized buffers, special values and bad
arguments.  Built with the host compilers (gcc / g++; no GPU code is
involved) and run here on the CPU; a sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _build_and_run(tmp_path, compiler, sources, extra, name):
    exe = str(tmp_path / name)
    cmd = [compiler, *SAN, *extra, "-o", exe, *sources, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{' '.join(cmd)}\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in report and "AddressSanitizer" not in report, report
    return report


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_oracle_under_asan_ubsan(tmp_path):
    out = _build_and_run(tmp_path, "gcc", [os.path.join(ROOT, "oracle", "kq_oracle.c"),
                                           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")],
                         ["-std=c11"], "oracle_san")
    assert "oracle driver ok" in out


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_host_helpers_under_asan_ubsan(tmp_path):
    out = _build_and_run(tmp_path, "g++", [os.path.join(ROOT, "mxfp4_act_quantizer_amd", "csrc", "kq_host.cpp"),
                                           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp")],
                         ["-std=c++17", "-I", os.path.join(ROOT, "include")], "host_san")
    assert "host driver ok" in out
