"""The oracle and the library's host-side validation under AddressSanitizer
and UndefinedBehaviorSanitizer (CPU only): builds both instrumented and runs
the CPU tests that use them, each library in its own process with its own
sanitizer runtime preloaded (oracle/sanitize_check.py)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs gcc and hipcc")
def test_sanitized_oracle_and_validation_run_clean():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "oracle", "sanitize_check.py")], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout and "failed" not in r.stdout
