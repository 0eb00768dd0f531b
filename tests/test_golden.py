"""Stored fixtures: the pages' printed facts and an oracle-written regression file."""
import json
import os

import numpy as np

import oracle
import workloads as wl
from tests.golden.make_golden import hash_arr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_tiny_probe_row_regression():
    # tiny_probe_row.txt was written by tests/golden/make_golden.py from the
    # oracle; inputs and outputs must both still reproduce bit for bit.
    w = wl.tiny_weights(0)
    with open(os.path.join(GOLDEN, "tiny_probe_row.txt")) as f:
        lines = f.read().splitlines()
    assert lines[1] == f"# input sha: probe={hash_arr(w.probes)} w={hash_arr(w.w)} b={hash_arr(w.b)}"
    bits = np.array([int(l.split()[1], 16) for l in lines[2:]], np.uint32)
    y = oracle.linear_f32(w.probes, w.w, w.b)[0]
    np.testing.assert_array_equal(y.view(np.uint32), bits)


def test_page_facts_are_what_the_suite_uses():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)
    assert facts["bitwise_m_sweep"]["value"] == [1, 8, 15, 16, 17, 32, 33, 64]
    assert set(facts["bitwise_m_sweep"]["value"]) <= set(wl.ROUTER_DECODE_M)
    assert (facts["router_shape"]["N"], facts["router_shape"]["K"]) == (wl.ROUTER_N, wl.ROUTER_K)
    assert facts["fp32_tolerance"]["atol"] == 2e-3 and facts["fp32_tolerance"]["rtol"] == 1e-4
