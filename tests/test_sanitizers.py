"""CPU sanitizer check (no GPU): builds the AddressSanitizer + UndefinedBehaviorSanitizer versions of
the oracle, the host input generator and the C-ABI library's host code (tests/sanitized.py) and runs
the ABI boundary tests and the oracle's layer pins (brute force, exact block sums, routing) with them
loaded.  The whole CPU suite runs the
same way with `python tests/sanitized.py`."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SCRIPT = os.path.join(HERE, "sanitized.py")


def test_abi_and_oracle_pins_under_asan_and_ubsan():
    if not os.path.exists(SCRIPT):
        pytest.skip("sanitizer build script not present")
    if not os.path.exists("/opt/rocm/llvm/bin/clang"):
        pytest.skip("ROCm clang not installed")
    r = subprocess.run([sys.executable, SCRIPT, os.path.join(HERE, "test_abi.py"),
                        os.path.join(HERE, "test_oracle_layer.py")], capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail, tail
