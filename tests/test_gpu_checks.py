"""The debug build with device-side index-range checks
(libmoe_mi355x_checks.so): no check fails on the kernel paths the parity
tests use, its outputs are bit-identical to the release build's, and a
dispatch given an out-of-range expert id sets MOE_CHECK_DISPATCH_ID (the
kernel skips that id in both builds, so nothing is accessed out of range).
The checks build runs in a process of its own (tests/checks_driver.py)."""

import json
import os
import subprocess
import sys

import pytest
import torch

from sparse_moe_layer_03_amd import binding as B
from tests import checks_driver as D

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_debug_checks_build_finds_no_violation_and_matches_release():
    assert os.path.exists(B.LIB_CHECKS_PATH), "build it with build(checks=True)"
    env = dict(os.environ, MOE_MI355X_LIB=B.LIB_CHECKS_PATH)
    p = subprocess.run([sys.executable, "-m", "tests.checks_driver"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=200)
    assert p.returncode == 0, p.stderr[-3000:]
    res = json.loads(p.stdout.strip().splitlines()[-1])
    print(res, flush=True)
    assert res["lib"] == os.path.basename(B.LIB_CHECKS_PATH)
    assert res["valid_bits"] == 0, [n for b, n in B.CHECK_BITS.items() if res["valid_bits"] & b]
    dispatch_id = next(b for b, n in B.CHECK_BITS.items() if n == "MOE_CHECK_DISPATCH_ID")
    assert res["invalid_bits"] == [dispatch_id, dispatch_id]
    # the release build (this process) computes the same bits
    for w in D.LAYER_CASES:
        assert D.layer_case(w) == res["digests"][w.name], w.name
    for d, dff in D.R320_CASES:
        assert D.r320_case(d, dff) == res["digests"][f"rows320_{d}_{dff}"], (d, dff)
    torch.cuda.synchronize()
