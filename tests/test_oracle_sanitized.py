"""The oracle's pin tests again, against a build of the oracle with AddressSanitizer and UBSan: no
out-of-bounds access and no undefined behaviour on any of their inputs (a report aborts the child run)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_formats.py", "tests/test_oracle_quant.py", "tests/test_oracle_products.py",
             "tests/test_oracle_b3.py"]


def _asan_runtime():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    except (OSError, subprocess.CalledProcessError):
        return None
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_asan_runtime() is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_oracle_pins_pass_under_sanitizers():
    env = dict(os.environ, LOWBIT_ORACLE_SANITIZE="1", LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([sys.executable, "-m", "pytest", *PIN_FILES, "-q", "-p", "no:cacheprovider"], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "failed" not in r.stdout
