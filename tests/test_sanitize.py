"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two drivers (tests/sanitize/) run against sanitizer builds:
  - abi_driver: every C entry point's host-side checks (pointers, sizes,
    offsets, segment arrays, ring arguments, overflow guards), the split
    heuristic over a grid of shapes and the status strings, linked against a
    copy of librattn whose host code is built with both sanitizers;
  - oracle_driver: every entry point of the fp64 CPU oracle over a sweep of
    shapes, dtypes, GQA groupings and causal offsets, with property checks
    (empty rows, convex combinations, merge of key halves, sum of dV).
A sanitizer report aborts the driver (-fno-sanitize-recover=all), so a clean
exit with status 0 is the pass.
"""
import os
import shutil
import subprocess

import pytest

from ring_attention_amd import build as rbuild

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or not os.path.exists(rbuild.hipcc()),
                                reason="needs gcc and hipcc")


@pytest.fixture(scope="module")
def drivers():
    return rbuild.build_sanitize_checks()


def run(path):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([path], capture_output=True, text=True, env=env, timeout=600)
    return r.returncode, r.stdout + r.stderr


def test_abi_host_checks_under_sanitizers(drivers):
    rc, out = run(drivers[0])
    assert rc == 0, out[-4000:]
    assert "0 failures" in out


def test_oracle_under_sanitizers(drivers):
    rc, out = run(drivers[1])
    assert rc == 0, out[-4000:]
    assert "0 failures" in out
