"""CPU checks of the parity report and bounds themselves (parity_util)."""

import numpy as np
import pytest

import oracle
from gqa_inputs import bf16_bits, decode_inputs, seed_base
from parity_util import TOL_MAX, TOL_MEAN, assert_close, bf16_ulp, check_close, compare


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


@pytest.fixture(scope="module")
def decode_64k_split():
    """The batch-1 64K-key decode (the workload's inputs) as the oracle's own split-KV pieces:
    32 chunks of 2048 keys, the split a GPU decode of this length uses."""
    q, kc, vc, lens = decode_inputs(1, 65536, base=seed_base(1, 5))
    o_part, lse = oracle.decode_partials(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), lens, 2048)
    want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), lens)
    return o_part, lse, want


def _as_gpu(x):
    """What a correct bf16 output of the same arithmetic would hold: x rounded to bf16."""
    return oracle.round_to_bf16(x)


def test_floor_bound_accepts_the_exact_merge(decode_64k_split):
    o_part, lse, want = decode_64k_split
    got = _as_gpu(oracle.combine_partials(o_part, lse))
    assert np.max(np.abs(oracle.combine_partials(o_part, lse) - want)) < 1e-12
    assert_close(got, want, "all 32 splits merged")


@pytest.mark.parametrize("dropped", [[5], [0, 9, 17, 31]])
def test_floor_bound_rejects_a_merge_missing_splits(decode_64k_split, dropped):
    o_part, lse, want = decode_64k_split
    lse = lse.copy()
    lse[..., dropped] = -np.inf              # those splits never arrived
    got = _as_gpu(oracle.combine_partials(o_part, lse))
    ok, msg, mx, mean = check_close(got, want, f"splits {dropped} dropped")
    print(msg)
    # the workload's stated tolerance alone would accept this result ...
    assert mx <= TOL_MAX and mean <= TOL_MEAN
    # ... the floor-relative bound does not
    assert not ok


def test_floor_bound_rejects_a_five_percent_scale_error(decode_64k_split):
    o_part, lse, want = decode_64k_split
    got = _as_gpu(1.05 * oracle.combine_partials(o_part, lse))
    ok, msg, mx, mean = check_close(got, want, "output scaled by 1.05")
    print(msg)
    assert mx <= TOL_MAX and mean <= TOL_MEAN
    assert not ok
