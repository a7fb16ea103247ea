"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the fp64 oracle (oracle/sdv_oracle.c, gcc) and the library's host HMAC-SHA-256 uniforms
(csrc/sdcp_uniforms.cpp, g++) with -fsanitize=address,undefined, then runs the oracle's pins and
the HMAC check (tests/sanitized_pins.py) against those builds in a child process.  Any report
aborts the child, which fails the test.  Host code only: nothing here touches a GPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime(name):
    cc = shutil.which("gcc")
    if cc is None:
        return None
    path = subprocess.run([cc, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_and_hmac_are_clean_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None or shutil.which("g++") is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    oracle_so = str(tmp_path / "liboracle_san.so")
    sdcp_so = str(tmp_path / "libsdcp_san.so")
    subprocess.run(["gcc", *SAN, "-std=c11", "-fopenmp", "-shared", "-fPIC",
                    os.path.join(ROOT, "oracle", "sdv_oracle.c"), "-o", oracle_so, "-lm"], check=True)
    subprocess.run(["g++", *SAN, "-std=c++17", "-shared", "-fPIC",
                    os.path.join(ROOT, "lossless_draft_verification_online_amd", "csrc", "sdcp_uniforms.cpp"),
                    "-o", sdcp_so], check=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    res = subprocess.run([sys.executable, os.path.join(HERE, "sanitized_pins.py"), oracle_so, sdcp_so], env=env,
                         capture_output=True, text=True, timeout=900)
    report = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, report
    assert "sanitized pins ok" in res.stdout, report
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, report
