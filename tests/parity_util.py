"""Shared helpers for the GPU parity tests: device transfer and error measures.

Two bounds, both over every compared element:
- the tolerance the workload states for a bf16 output compared with an fp64
  reference: max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3;
- a bound relative to the rounding floor, the error the oracle itself makes when its
  result is rounded to bf16 (the least any bf16 output can have): max error <= 4x and
  mean error <= 2x the floor's. At long contexts the outputs are small (|out| ~ 0.03 at
  64K keys), the floor is ~6e-5, and the stated tolerance alone would pass a decode
  that lost a split of its cache; the floor-relative bound does not
  (tests/test_parity_util.py plants such mistakes in the oracle's own split merge).
"""

import numpy as np
import torch

import oracle
from gqa_inputs import bf16_bits

TOL_MAX = 2e-2
TOL_MEAN = 2e-3
FLOOR_MAX_FACTOR = 4.0
FLOOR_MEAN_FACTOR = 2.0


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda:0").contiguous()


def gpu_f64(t: torch.Tensor) -> np.ndarray:
    """bf16 GPU tensor -> float64 numpy (exact)."""
    return oracle.bf16_bits_to_f64(bf16_bits(t))


def errors(got: np.ndarray, want: np.ndarray):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU output"
    d = np.abs(got - want)
    return float(d.max()), float(d.mean())


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significand bits); the smallest normal's for 0."""
    a = np.maximum(np.abs(x), np.float64(2.0) ** -126)
    return np.float64(2.0) ** (np.floor(np.log2(a)) - 7)


def compare(got: np.ndarray, want: np.ndarray) -> dict:
    """Diagnostic report of a GPU result against the fp64 oracle: error measures, NaN/Inf
    counts, the first element past TOL_MAX (flat index) and a histogram of the distance
    to the oracle's own bf16 rounding, in bf16 ulps of that rounded value."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    d = np.abs(got - want)
    r = oracle.round_to_bf16(want)
    ulps = np.abs(got - r) / bf16_ulp(r)
    bad = np.flatnonzero(~(d <= TOL_MAX))
    edges = [0, 1, 2, 4, 16]
    hist = {"0": int(np.sum(ulps == 0))}
    for lo, hi in zip(edges[:-1], edges[1:]):
        hist[f"({lo},{hi}]"] = int(np.sum((ulps > lo) & (ulps <= hi)))
    hist[f">{edges[-1]}"] = int(np.sum(ulps > edges[-1]))
    rel = d / np.maximum(np.abs(want), 1e-6)
    return {
        "n": int(d.size), "max_abs": float(np.nanmax(d)) if d.size else 0.0,
        "mean_abs": float(np.nanmean(d)) if d.size else 0.0,
        "max_rel_where_abs_ge_1e-2": float(np.max(rel[np.abs(want) >= 1e-2])) if np.any(np.abs(want) >= 1e-2) else 0.0,
        "nan": int(np.isnan(got).sum()), "inf": int(np.isinf(got).sum()),
        "first_past_tol": int(bad[0]) if bad.size else None,
        "ulp_hist_vs_bf16_oracle": hist,
    }


def check_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    """(ok, message): both bounds of the module docstring. Where the oracle's result is
    exactly representable in bf16 everywhere (floor 0), only the stated tolerance applies;
    such cases carry exact checks of their own."""
    mx, mean = errors(got, want)
    floor_mx, floor_mean = errors(oracle.round_to_bf16(want), want)
    rep = compare(got, want)
    ok_tol = mx <= TOL_MAX and mean <= TOL_MEAN
    if floor_mx > 0:
        ok_floor = mx <= FLOOR_MAX_FACTOR * floor_mx and mean <= FLOOR_MEAN_FACTOR * floor_mean
        ratio = f"{mx / floor_mx:.2f}x / {mean / floor_mean:.2f}x (bound {FLOOR_MAX_FACTOR}x / {FLOOR_MEAN_FACTOR}x)"
    else:
        ok_floor = True
        ratio = "n/a (oracle exact in bf16)"
    msg = (f"{what}: max abs err {mx:.3e} (tol {TOL_MAX}), mean {mean:.3e} (tol {TOL_MEAN}); "
           f"bf16 rounding floor max {floor_mx:.3e} mean {floor_mean:.3e}; error / floor {ratio}; "
           f"ulps vs bf16(oracle) {rep['ulp_hist_vs_bf16_oracle']}")
    return ok_tol and ok_floor, msg, mx, mean


def assert_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    ok, msg, mx, mean = check_close(got, want, what)
    print(msg, flush=True)
    assert ok, msg
    return mx, mean


def sample_rows(S: int, extra: int = 16, seed: int = 0):
    """Query rows to check at full size: both ends, tile and wave boundaries, the middle,
    plus a few random ones."""
    base = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, S // 2 - 1, S // 2, S - 65, S - 64,
            S - 33, S - 32, S - 2, S - 1]
    rng = np.random.default_rng(seed)
    rnd = rng.integers(0, S, size=extra).tolist()
    return sorted({r for r in base + rnd if 0 <= r < S})
