"""Prefill parity for the two workgroup forms beside the 4-wave one.

The 8-wave form (two 32-row blocks per head, a 4-stage K/V ring published two tiles per
barrier) is taken once its grid holds at least 5/3 workgroups per CU; the key-split form
(4 units of two waves each, every wave streaming half of its unit's key tiles, merged by
log-sum-exp weights) when the 4-wave grid holds at most 2. Every case first asserts,
through gqa.prefill_plan, that the shape really runs the form under test, then checks it
against the oracle (full compare, or sampled rows at the larger sizes). A batch run
through the 8-wave kernel must also equal, bit for bit, its sequences run one at a time
through the 4-wave kernel: both forms give each wave the same rows and the same
operation order."""

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
    (1, 3500, 32, 8, True, True),       # batch 1 just past the 4-wave range, ragged tail
    (8, 1000, 32, 8, True, True),
    (8, 1000, 32, 8, False, True),
    (64, 130, 32, 8, True, False),      # ragged last tile, 5 row blocks per head
    (32, 777, 8, 8, True, True),        # G = 1
    (8, 1000, 48, 8, True, True),       # G = 6: row blocks of two heads share a workgroup
    (8, 640, 64, 4, False, True),       # G = 16
]


@pytest.mark.parametrize("B,S,Hq,Hkv,causal,sampled", CASES)
def test_prefill_8wave_matches_oracle(B, S, Hq, Hkv, causal, sampled):
    waves, wgs, ks = gqa.prefill_plan(B, S, Hq, Hkv)
    _say(f"prefill 8-wave B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}: plan {waves} waves, {wgs} workgroups")
    assert (waves, ks) == (8, 1)
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
    B, S = 16, 500
    assert gqa.prefill_plan(B, S, 32, 8) == (8, 16 * 8 * 8, 1)
    assert gqa.prefill_plan(1, S, 32, 8) == (4, 8 * 16, 1)
    _say(f"prefill B={B} S={S} causal={causal}: 8-wave batch vs 4-wave per sequence, bitwise")
    q, k, v = [dev(x) for x in prefill_inputs(B, S, base=7700 + int(causal))]
    batch = gqa.prefill(q, k, v, causal=causal)
    one = torch.cat([gqa.prefill(q[b:b + 1], k[b:b + 1], v[b:b + 1], causal=causal) for b in range(B)])
    torch.cuda.synchronize()
    assert torch.equal(batch.view(torch.int16), one.view(torch.int16))


# (B, S, Hq, Hkv, causal, rows sampled?): key-split shapes. Odd and even tile counts, a
# ragged last tile, workgroups whose second half gets no tile (the first query tiles of a
# causal run), and the group sizes of the other tests.
SPLIT_CASES = [
    (1, 512, 32, 8, True, False),       # 8 tiles in the longest job, 4 per half
    (1, 520, 32, 8, False, False),      # 9 tiles: 5 + 4, ragged last tile
    (1, 1000, 32, 8, True, True),
    (1, 2048, 32, 8, True, True),       # largest B = 1 shape of this form
    (1, 2048, 32, 8, False, True),
    (2, 777, 32, 8, True, True),
    (1, 1500, 8, 8, True, True),        # G = 1
    (1, 1000, 48, 8, True, True),       # G = 6
    (1, 900, 64, 4, False, True),       # G = 16
]


@pytest.mark.parametrize("B,S,Hq,Hkv,causal,sampled", SPLIT_CASES)
def test_prefill_key_split_matches_oracle(B, S, Hq, Hkv, causal, sampled):
    waves, wgs, ks = gqa.prefill_plan(B, S, Hq, Hkv)
    _say(f"prefill key-split B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}: plan {waves} waves, {wgs} workgroups")
    assert (waves, ks) == (8, 2)
    q, k, v = prefill_inputs(B, S, Hq, Hkv, D, base=7800 + B + S + Hq)
    out = gqa.prefill(dev(q), dev(k), dev(v), causal=causal)
    torch.cuda.synchronize()
    if sampled:
        rows = sample_rows(S, seed=S + Hq)   # includes the shortest and the longest jobs
        for b in sorted({0, B - 1}):
            got = gpu_f64(out[b:b + 1, rows])
            want = oracle.prefill(bf16_bits(q[b:b + 1]), bf16_bits(k[b:b + 1]), bf16_bits(v[b:b + 1]),
                                  causal=causal, rows=rows)
            assert_close(got, want, f"key-split B={B} S={S} Hq={Hq} Hkv={Hkv} batch element {b}")
    else:
        got = gpu_f64(out)
        want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=causal)
        assert_close(got, want, f"key-split B={B} S={S} Hq={Hq} Hkv={Hkv}")


# Every form with the scales that take the kernels' other code paths: zero and negative
# scales (the scale is then applied to the scores before the row max) and a large one.
FORM_SHAPES = {"4-wave": (1, 300, (4, 1)), "key-split": (1, 600, (8, 2)), "8-wave": (8, 600, (8, 1))}


@pytest.mark.parametrize("form", sorted(FORM_SHAPES))
@pytest.mark.parametrize("scale", [0.0, -0.0883883461356163, 0.5])
def test_every_form_with_other_scales(form, scale):
    B, S, want_plan = FORM_SHAPES[form]
    waves, wgs, ks = gqa.prefill_plan(B, S, 32, 8)
    _say(f"prefill {form} B={B} S={S} scale={scale}: plan {waves} waves, {ks} key splits")
    assert (waves, ks) == want_plan
    q, k, v = prefill_inputs(B, S, base=7900 + S)
    out = gqa.prefill(dev(q), dev(k), dev(v), causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = sample_rows(S, seed=S)
    for b in sorted({0, B - 1}):
        got = gpu_f64(out[b:b + 1, rows])
        want = oracle.prefill(bf16_bits(q[b:b + 1]), bf16_bits(k[b:b + 1]), bf16_bits(v[b:b + 1]),
                              causal=True, scale=scale, rows=rows)
        assert_close(got, want, f"{form} scale={scale} batch element {b}")


def test_8wave_form_with_idle_waves():
    # S = 1 at B = 64: 8-wave workgroups whose second row block does not exist, so waves
    # 4-7 stream no tile of their own; a single key must still give V[0] exactly
    B = 64
    assert gqa.prefill_plan(B, 1, 32, 8)[0] == 8
    _say(f"prefill 8-wave B={B} S=1: out == V[0] bitwise")
    q, k, v = prefill_inputs(B, 1, base=7950, sigma_qk=16.0)
    out = gqa.prefill(dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    want = v.repeat_interleave(4, dim=2)          # query head h reads KV head h // 4
    assert torch.equal(out.cpu().view(torch.int16), want.view(torch.int16))
    # S = 40: a partial second row block and a ragged single tile
    B, S = 64, 40
    assert gqa.prefill_plan(B, S, 32, 8)[0] == 8
    _say(f"prefill 8-wave B={B} S={S} against the oracle")
    q, k, v = prefill_inputs(B, S, base=7951)
    out = gqa.prefill(dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    for b in (0, B - 1):
        got = gpu_f64(out[b:b + 1])
        want = oracle.prefill(bf16_bits(q[b:b + 1]), bf16_bits(k[b:b + 1]), bf16_bits(v[b:b + 1]), causal=True)
        assert_close(got, want, f"8-wave B={B} S={S} batch element {b}")


# Every form at shapes the library would not pick it for (through gqa_attn_prefill_form):
# short and long prompts, ragged tails, batches, non-causal, other head groupings.
# (B, S, Hq, Hkv, causal)
FORM_CASES = [
    (1, 100, 32, 8, True),       # one key tile per unit: the key split's second half is empty
    (1, 700, 32, 8, True),
    (1, 4200, 32, 8, True),      # the key split where the library runs 8 waves
    (2, 1500, 32, 8, False),
    (3, 333, 8, 8, True),        # G = 1
    (2, 900, 48, 8, True),       # G = 6
]


@pytest.mark.parametrize("form", gqa.PREFILL_FORMS)
@pytest.mark.parametrize("B,S,Hq,Hkv,causal", FORM_CASES)
def test_every_form_at_shapes_it_is_not_chosen_for(form, B, S, Hq, Hkv, causal):
    _say(f"prefill form={form} B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}; plan {gqa.prefill_plan(B, S, Hq, Hkv)}")
    q, k, v = prefill_inputs(B, S, Hq, Hkv, D, base=7900 + B + S + Hq)
    out = gqa.prefill(dev(q), dev(k), dev(v), causal=causal, form=form)
    torch.cuda.synchronize()
    rows = sample_rows(S, seed=S + B) if S > 1024 else None
    for b in range(B):
        got = gpu_f64(out[b:b + 1] if rows is None else out[b:b + 1, rows])
        want = oracle.prefill(bf16_bits(q[b:b + 1]), bf16_bits(k[b:b + 1]), bf16_bits(v[b:b + 1]),
                              causal=causal, rows=rows)
        assert_close(got, want, f"form={form} B={B} S={S} Hq={Hq} Hkv={Hkv} batch element {b}")
    if form == (8, 1):
        ref = gqa.prefill(dev(q), dev(k), dev(v), causal=causal, form=(4, 1))
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
