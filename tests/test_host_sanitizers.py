"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/host_driver.cpp drives every entry point's argument checks, the
workspace arithmetic and the host pairing (Theorem 4.2) against brute force; it is
compiled together with the library's sources (the sanitizers apply to the host code
alone: every -fsanitize= is passed with -Xarch_host; no GPU code is launched) and
run on the CPU. Any sanitizer report or failed check fails the test.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

from sparse_decode_attention_saga_amd import build as build_mod

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "sanitize", "host_driver.cpp")


@pytest.mark.skipif(not os.path.exists(build_mod.hipcc()), reason="hipcc is not installed")
def test_host_code_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "host_driver")
        cmd = [build_mod.hipcc(), f"--offload-arch={build_mod.ARCH}", "-x", "hip", "-O1", "-Xarch_host", "-g",
               "-std=c++17", "-Xarch_host", "-fno-omit-frame-pointer",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined",
               "-I", os.path.join(build_mod.ROOT, "include"), "-o", exe] + build_mod.SOURCES + [DRIVER]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-4000:]
        # the sanitizers really are in the host code
        syms = subprocess.run(["nm", exe], capture_output=True, text=True).stdout
        assert "__asan_init" in syms and "__ubsan_handle_" in syms
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        out = run.stdout + run.stderr
        assert run.returncode == 0, out[-4000:]
        assert "host checks: 0 failed" in out
        assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
