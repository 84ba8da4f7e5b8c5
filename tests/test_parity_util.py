"""CPU checks of the parity report itself (parity_util.compare)."""

import numpy as np

import oracle
from parity_util import bf16_ulp, compare


def test_ulp_spacing():
    assert bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert bf16_ulp(np.array([-3.0]))[0] == 2.0 ** -6
    assert bf16_ulp(np.array([0.0]))[0] == 2.0 ** -133


def test_compare_histogram_and_first_index():
    want = np.linspace(0.1, 0.9, 101)
    r = oracle.round_to_bf16(want)
    rep = compare(r, want)
    assert rep["ulp_hist_vs_bf16_oracle"]["0"] == 101 and rep["first_past_tol"] is None
    one = r + bf16_ulp(r)                 # exactly one ulp above the oracle's rounding
    assert compare(one, want)["ulp_hist_vs_bf16_oracle"]["(0,1]"] == 101
    bad = r.copy()
    bad[37] += 0.05
    bad[80] = np.nan
    rep = compare(bad, want)
    assert rep["first_past_tol"] == 37 and rep["nan"] == 1
