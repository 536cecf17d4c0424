"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/sanitize_host.cpp drives the CPU side of the hybrid layer (pi_cold_ffn_ex on
both code paths and several thread counts, pi_host_read_probe) and the oracle's
functions over seeded inputs of small, ragged shapes, with the host operator
checked against the oracle.  Both libraries' sources are compiled here with g++ /
gcc and -fsanitize=address,undefined (host code only; no GPU code is built), and
any report or out-of-bound result fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1",
       "-fopenmp", "-ffp-contract=off"]


def _run(cmd, **kw):
    return subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)


def test_host_code_under_sanitizers(tmp_path):
    if not (shutil.which("g++") and shutil.which("gcc")):
        pytest.skip("no host compiler")
    obj = str(tmp_path / "oracle.o")
    r = _run(["gcc", *SAN, "-std=c11", "-c", os.path.join(ROOT, "oracle", "oracle.c"), "-o", obj])
    if r.returncode != 0 and ("asan" in r.stdout or "ubsan" in r.stdout):
        pytest.skip("sanitizer runtime not available: " + r.stdout[-300:])
    assert r.returncode == 0, r.stdout
    exe = str(tmp_path / "sanitize_host")
    r = _run(["g++", *SAN, "-std=c++17", os.path.join(ROOT, "tests", "sanitize_host.cpp"),
              os.path.join(ROOT, "activation_sparse_amd", "csrc", "pi_host.cpp"), obj, "-o", exe])
    assert r.returncode == 0, r.stdout
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="8")
    r = _run([exe], env=env, timeout=600)
    assert r.returncode == 0 and "clean" in r.stdout, r.stdout[-4000:]
