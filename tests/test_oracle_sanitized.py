"""The oracle's pins run again against a build of the oracle under
AddressSanitizer and UndefinedBehaviorSanitizer (including float-to-integer
conversions out of range), every report fatal: out-of-bounds accesses,
undefined conversions (a NaN turned into a code) and the like fail here even
where the plain build happens to give the expected bits.  Host code only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_pins.py", "tests/test_norm_pins.py", "tests/test_rotation_pins.py",
             "tests/test_quality_pins.py"]


def _libasan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = build.build_sanitized(str(tmp_path / "libsq_oracle_san.so"))
    env = dict(os.environ, SQ_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
