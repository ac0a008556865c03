"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C-ABI runtime (argument checks, the tuning-table JSON parser and lookup,
workspace bookkeeping) and the fp64 oracle are rebuilt with
-fsanitize=address,undefined, and the host-side suites run against those
builds in a subprocess with libasan preloaded: the ABI checks, the tuner's
host logic and the oracle's pins.  A planted heap overflow in a throwaway
library shows that the harness reports what it should."""
import os
import subprocess
import sys

import pytest

import oracle
from swiglu_mlp_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_env(**extra):
    env = dict(os.environ)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **extra)
    return env


def _have(tool):
    from shutil import which
    return which(tool) is not None


pytestmark = pytest.mark.skipif(not (_have("gcc") and _have("g++")), reason="needs gcc/g++")


def test_harness_catches_a_planted_overflow(tmp_path):
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint poke(int n) { int *p = malloc(4 * n); p[n] = 1; int v = p[0];"
                   " free(p); return v; }\n")
    lib = tmp_path / "libbad.so"
    subprocess.run(["gcc", "-shared", "-fPIC", "-g", "-fsanitize=address", str(src), "-o", str(lib)], check=True)
    code = f"import ctypes; ctypes.CDLL({str(lib)!r}).poke(4)"
    r = subprocess.run([sys.executable, "-c", code], env=_asan_env(), capture_output=True, text=True)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_host_suites_under_asan_ubsan(tmp_path):
    lib = hip_build.build_host_sanitized(str(tmp_path / "libdfk_san.so"))
    orc = oracle.build(oracle.SOURCE, str(tmp_path / "liboracle_san.so"),
                       extra=["-g", "-fno-omit-frame-pointer", *hip_build.SANITIZE])
    tests = [os.path.join(ROOT, "tests", t) for t in ("test_abi.py", "test_tuner_host.py", "test_oracle_pins.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *tests],
                       env=_asan_env(DFK_LIBRARY=lib, DFK_ORACLE_LIBRARY=orc), cwd=ROOT,
                       capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
