"""The C-ABI CPU tests (plans, layouts, validation and error paths, the
unbounded request) against a build whose host code runs under
AddressSanitizer and UndefinedBehaviorSanitizer: any out-of-bounds access,
use after free or undefined behaviour in the host library aborts the run.
The concern is the host bookkeeping of slots and plans across rounds (WF
App. B.2 Eq. 13 double buffer, App. B.3 promotion), exercised here over
every round of hundreds of configs."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_abi_cpu_tests_pass_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from chunk_causal_dit_round_amd.build_sanitized import asan_runtime, build_sanitized

    lib = build_sanitized()
    env = dict(os.environ)
    env.update(WF_LIBRARY=lib, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-p", "no:xdist", os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail, tail
