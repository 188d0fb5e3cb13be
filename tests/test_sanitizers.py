"""The CPU suite under AddressSanitizer + UBSan builds of the oracle and of libpa's host code.

tests/sanitize.py builds both into a temporary directory, checks that each carries
sanitizer calls, and runs the `-m "not gpu"` tests in child processes with the
matching runtime preloaded; any report fails the child and so this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("nm") is None,
                    reason="gcc and nm are needed for the sanitizer builds")
@pytest.mark.parametrize("which", ["oracle", "host"])
def test_cpu_suite_passes_under_sanitizers(which):
    if which == "host" and not os.path.exists("/opt/rocm/bin/hipcc") and not shutil.which("hipcc"):
        pytest.skip("hipcc is needed for the host-sanitized libpa")
    res = subprocess.run([sys.executable, os.path.join(HERE, "sanitize.py"), which],
                         capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert " passed" in res.stdout and "ERROR: AddressSanitizer" not in tail, tail
