"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): oracle/build.py --sanitize builds the same C source with both
(every report fatal), and a child interpreter with the sanitizer runtimes
preloaded runs the pin suites against that build.  Any out-of-bounds access,
use after free, signed overflow, misaligned access or other undefined
behaviour in the oracle ends the child with a report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_margins.py", "tests/test_oracle_law.py"]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build(sanitize=True)
    assert os.path.exists(lib)
    env = build.sanitizer_env()
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not slow",
                        *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
