"""The host-side argument checks and launch planning under the address and
undefined-behaviour sanitizers: a seeded random driver (csrc/validate_check.cpp)
feeds every plan function edge-case arguments and checks the invariants of the
plans it accepts.  CPU only."""
import os
import re
import shutil
import subprocess

import pytest

from exact_attention_43_amd import build

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


@pytest.fixture(scope="module")
def checker():
    return build.build_host_checker()


@pytest.mark.parametrize("seed", [1, 2])
def test_plans_under_sanitizers(checker, seed):
    env = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    r = subprocess.run([checker, "300000", str(seed)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
    counts = {m.group(1): (int(m.group(2)), int(m.group(3)))
              for m in re.finditer(r"^(\w+)\s+accepted\s+(\d+)\s+rejected\s+(\d+)$", r.stdout, re.M)}
    assert set(counts) == {"plan_fwd", "plan_fwd_fp8", "plan_decode", "check_append", "check_paged",
                           "plan_bwd", "auto_splits", "slot_schedule"}
    for name, (ok, rejected) in counts.items():
        # the draws reach both outcomes of every check
        assert ok > 100 and rejected > 100, (name, ok, rejected)
