"""The host-only code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds tests/sanitize_driver.cpp with g++ together with the library's
shape-only planner (conv_plan.cpp, which includes no HIP header, so it is
compiled here as plain C++) and the fp64 oracle (oracle/oracle.c), with
-fsanitize=address,undefined and no recovery, and runs it: seeded random
problems (sizes up to and beyond the int64 and 2^31-element limits) through
extents, auto_pad, plan, describe, scratch and check, compared with the
oracle's integer results; and the oracle's two formulations of Conv and
ConvTranspose on exact-size heap arrays.  Any overflow, wrap or out-of-bounds
access aborts the driver and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "convolution_forward_amd", "csrc")


def _build(tmp_path):
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("no host compiler")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    objs = []
    orc = str(tmp_path / "oracle.o")
    subprocess.check_call(["gcc", "-std=c11", "-c", *san, "-fopenmp",
                           os.path.join(ROOT, "oracle", "oracle.c"), "-o", orc])
    objs.append(orc)
    for src in sorted(os.listdir(CSRC)):
        if src.endswith(".cpp") and src != "conv_host.cpp":
            o = str(tmp_path / (src + ".o"))
            subprocess.check_call(["g++", "-std=c++17", "-c", *san, "-I", os.path.join(ROOT, "include"),
                                   "-I", CSRC, os.path.join(CSRC, src), "-o", o])
            objs.append(o)
    exe = str(tmp_path / "sanitize_driver")
    subprocess.check_call(["g++", "-std=c++17", *san, "-fopenmp", "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "sanitize_driver.cpp"), *objs, "-o", exe, "-lm"])
    return exe


def test_host_code_under_asan_ubsan(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="1")
    r = subprocess.run([exe, "20000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert "no failures" in r.stdout
