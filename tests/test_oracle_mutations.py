"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle and its pin tests into a temporary directory,
plants one mistake in the copy's source (at every place the mutated line occurs): a
wrong KV-head map, an off-by-one at the causal boundary, a flipped sign, a dropped
scale, a biased output, a wrong lens clamp, a broken combine weight, a wrong bf16
widening, reversed key dimensions, the causal mask applied to a full prefill, values
read from the wrong KV head, a partial's log-sum-exp in the wrong base, a split chunk
one key short, and a softmax without its max subtraction. It runs the pins on the copy
in a subprocess and expects them to fail. The real oracle is never touched.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("head_map_modulo", "return h // (Hq // Hkv)", "return h % Hkv"),
    ("causal_off_by_one", "x[ri, i + 1:] = -np.inf", "x[ri, i + 2:] = -np.inf"),
    ("softmax_sign", "e = np.exp(x - m)", "e = np.exp(m - x)"),
    ("scale_dropped", "x = s * (q[b, r, h, :] @ Kg[:nvis].T)", "x = (q[b, r, h, :] @ Kg[:nvis].T)"),
    ("decode_bias", "out[b, h, :] = p @ Vb[:, g, :]", "out[b, h, :] = p @ Vb[:, g, :] * 1.0001"),
    ("lens_clamp", "n = int(min(max(lens[b], 0), L))", "n = int(min(max(lens[b], 1), L))"),
    ("combine_weights", "w = np.where(finite, np.exp(np.where(finite, lse, 0.0) - Msafe), 0.0)",
     "w = np.where(finite, 1.0, 0.0)"),
    ("bf16_shift", "(b.astype(np.uint32) << np.uint32(16))", "(b.astype(np.uint32) << np.uint32(15))"),
    ("decode_key_dims_reversed", "x = s * (Kb[:, g, :] @ q[b, h, :])", "x = s * (Kb[:, g, ::-1] @ q[b, h, :])"),
    ("noncausal_treated_as_causal", "nvis = int(r.max()) + 1 if causal else S", "nvis = int(r.max()) + 1"),
    ("value_head_shifted", "Vg = v[b, :, g, :]", "Vg = v[b, :, (g + 1) % Hkv, :]"),
    ("lse_in_log2", "lse[b, h, c] = m + np.log(tot)", "lse[b, h, c] = m + np.log2(tot)"),
    ("chunk_end_short", "j0, j1 = c * chunk, min((c + 1) * chunk, n)", "j0, j1 = c * chunk, min((c + 1) * chunk - 1, n)"),
    ("max_not_subtracted", "e = np.exp(x - m)", "e = np.exp(x)"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_the_pins(tmp_path, name, old, new):
    for d in ("oracle", "gqa_inputs"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests" / "golden").mkdir(parents=True)
    shutil.copy(os.path.join(ROOT, "tests", "test_oracle_pins.py"), tmp_path / "tests")
    shutil.copy(os.path.join(ROOT, "tests", "conftest.py"), tmp_path / "tests")
    shutil.copy(os.path.join(ROOT, "tests", "golden", "closed_form_cases.json"), tmp_path / "tests" / "golden")
    src_path = tmp_path / "oracle" / "attention.py"
    src = src_path.read_text()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    src_path.write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"
