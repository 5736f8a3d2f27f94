"""CPU checks of the oracle itself beyond its pins:

- its fp32 -> E4M3 encoder against an independent nearest-code search on every
  finite fp32 bit pattern (tests/e4m3_exhaustive.c, compiled with gcc);
- every oracle pin test (tests/test_oracle_*.py) run again, in a child
  process, against a build of oracle.c instrumented with AddressSanitizer and
  UndefinedBehaviorSanitizer (host code only; gcc), so that an out-of-bounds
  access or undefined arithmetic in the oracle fails the suite."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
GCC = shutil.which("gcc")

pytestmark = pytest.mark.skipif(GCC is None, reason="gcc is needed to build the checks")


def test_e4m3_encoder_on_every_finite_fp32(tmp_path):
    exe = str(tmp_path / "e4m3_exhaustive")
    subprocess.run([GCC, "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-I", ORACLE, os.path.join(ROOT, "tests", "e4m3_exhaustive.c"),
                    os.path.join(ORACLE, "oracle.c"), "-lm", "-o", exe], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checked 4278190080 finite fp32 patterns, 0 mismatches" in r.stdout


def _runtime(name):
    path = subprocess.run([GCC, f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not installed")
    return path


def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.run([GCC, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-o", lib,
                    os.path.join(ORACLE, "oracle.c"), "-lm"], check=True)
    env = dict(os.environ,
               LD_PRELOAD=" ".join([_runtime("libasan.so"), _runtime("libubsan.so")]),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               ORACLE_LIB=lib)
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    assert len(pins) >= 5
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *pins], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=1800)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
