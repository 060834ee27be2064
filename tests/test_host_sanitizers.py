"""The host code of the library (argument checks, workspace layout, status strings, the planner's host budget
with its radix sort) under AddressSanitizer and UndefinedBehaviorSanitizer: build.py --sanitize builds the
library with the host side instrumented (device code as usual) and runs the CPU ABI and host-budget tests
against it in a child process with the ASan runtime preloaded. Any report aborts that process."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_abi_and_host_budget_clean_under_asan_ubsan():
    r = subprocess.run([sys.executable, "-m", "draft_verification_acceptance_amd.build", "--sanitize",
                        "tests/test_abi.py", "tests/test_plan_host.py", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-3000:]
    assert "passed" in r.stdout and "failed" not in r.stdout
