"""The host C code under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/oracle.c and synth/synth.c are built again with
-fsanitize=address,undefined (every finding fatal), and the oracle pins and
the generator tests run against those builds in a child process, which
loads them through ORACLE_LIB / SYNTH_LIB with the sanitizer runtime
preloaded.  Host-only: no GPU is touched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _build(src, dst):
    cmd = ["gcc", *SAN, "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", dst, src, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)


def test_oracle_and_synth_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    orc = str(tmp_path / "liboracle_san.so")
    syn = str(tmp_path / "libsynth_san.so")
    _build(os.path.join(ROOT, "oracle", "oracle.c"), orc)
    _build(os.path.join(ROOT, "synth", "synth.c"), syn)
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ORACLE_LIB=orc, SYNTH_LIB=syn, OMP_NUM_THREADS="2",
               # the interpreter's own allocations are not leaks of the code under test
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_oracle_pins.py"),
           os.path.join(ROOT, "tests", "test_synth.py")]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
