"""Prefill parity for the 8-wave workgroup form (two 32-row blocks per head, a 4-stage
K/V ring published two tiles per barrier), which the library takes once its grid holds
at least 4 workgroups per CU. Every case first asserts, through gqa.prefill_plan, that
the shape really runs the 8-wave kernel, then checks it against the oracle (full
compare, or sampled rows at the larger sizes). A batch run through the 8-wave kernel
must also equal, bit for bit, its sequences run one at a time through the 4-wave
kernel: both forms give each wave the same rows and the same operation order."""

import pytest
import torch

import gqa_flash_attention_amd as gqa
import oracle
from gqa_inputs import D, bf16_bits, prefill_inputs
from parity_util import assert_close, dev, gpu_f64, sample_rows

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


# (B, S, Hq, Hkv, causal, rows sampled?)
CASES = [
    (8, 1000, 32, 8, True, True),
    (8, 1000, 32, 8, False, True),
    (64, 130, 32, 8, True, False),      # ragged last tile, 5 row blocks per head
    (32, 777, 8, 8, True, True),        # G = 1
    (8, 1000, 48, 8, True, True),       # G = 6: row blocks of two heads share a workgroup
    (8, 640, 64, 4, False, True),       # G = 16
]


@pytest.mark.parametrize("B,S,Hq,Hkv,causal,sampled", CASES)
def test_prefill_8wave_matches_oracle(B, S, Hq, Hkv, causal, sampled):
    waves, wgs = gqa.prefill_plan(B, S, Hq, Hkv)
    _say(f"prefill 8-wave B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}: plan {waves} waves, {wgs} workgroups")
    assert waves == 8
    q, k, v = prefill_inputs(B, S, Hq, Hkv, D, base=7600 + B + S + Hq)
    out = gqa.prefill(dev(q), dev(k), dev(v), causal=causal)
    torch.cuda.synchronize()
    if sampled:
        rows = sample_rows(S, seed=S + Hq)
        for b in (0, B // 2, B - 1):
            got = gpu_f64(out[b:b + 1, rows])
            want = oracle.prefill(bf16_bits(q[b:b + 1]), bf16_bits(k[b:b + 1]), bf16_bits(v[b:b + 1]),
                                  causal=causal, rows=rows)
            assert_close(got, want, f"8-wave B={B} S={S} Hq={Hq} Hkv={Hkv} batch element {b}")
    else:
        got = gpu_f64(out)
        want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=causal)
        assert_close(got, want, f"8-wave B={B} S={S} Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_8wave_equals_4wave_bitwise(causal):
    B, S = 16, 520
    assert gqa.prefill_plan(B, S, 32, 8)[0] == 8
    assert gqa.prefill_plan(1, S, 32, 8)[0] == 4
    _say(f"prefill B={B} S={S} causal={causal}: 8-wave batch vs 4-wave per sequence, bitwise")
    q, k, v = [dev(x) for x in prefill_inputs(B, S, base=7700 + int(causal))]
    batch = gqa.prefill(q, k, v, causal=causal)
    one = torch.cat([gqa.prefill(q[b:b + 1], k[b:b + 1], v[b:b + 1], causal=causal) for b in range(B)])
    torch.cuda.synchronize()
    assert torch.equal(batch.view(torch.int16), one.view(torch.int16))
