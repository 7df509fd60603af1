"""Sanitizer tier (CPU only): the oracle's pins and planted-mistake checks run
again against an AddressSanitizer + UndefinedBehaviorSanitizer build of
oracle/loki_oracle.c, in a child process with the sanitizer runtimes
preloaded; any out-of-bounds access, use after free or undefined behaviour
in the oracle aborts the child.  A first check plants an out-of-bounds read
in a throwaway library built the same way, to show the setup catches one.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def env():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not found")
    d = tempfile.mkdtemp(prefix="oracle_san_")
    lib = os.path.join(d, "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", *SAN, "-o",
                    lib, os.path.join(ROOT, "oracle", "loki_oracle.c"), "-lm"], check=True)
    e = dict(os.environ)
    e.update(LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
             UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", LOKI_ORACLE_LIB=lib,
             OMP_NUM_THREADS="4")
    return {"dir": d, "env": e}


def test_sanitizer_catches_a_planted_out_of_bounds_read(env):
    src = os.path.join(env["dir"], "oob.c")
    lib = os.path.join(env["dir"], "liboob.so")
    with open(src, "w") as f:
        f.write("#include <stdlib.h>\n"
                "int oob(int n) { int *a = malloc(n * sizeof(int)); for (int i = 0; i < n; i++)"
                " a[i] = i; int s = a[n]; free(a); return s; }\n")
    subprocess.run(["gcc", "-O0", "-g", "-fPIC", "-shared", *SAN, "-o", lib, src], check=True)
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({lib!r}).oob(8)"],
                       env=env["env"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr


def test_oracle_pins_under_sanitizers(env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_mutations.py")],
                       env=env["env"], capture_output=True, text=True, timeout=900, cwd=ROOT)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout
    assert "Sanitizer" not in r.stderr, tail
