"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test ties the oracle to something other than its own code: a pure-Python
brute force, an independent library routine (torch SDPA in float64), a closed
form, a hand-derived worked example, or an invariant of the definition of
softmax attention. Each is chosen so that a plausible slip (a dropped term, a
wrong sign, an off-by-one at the causal boundary, a wrong KV-head map, a
transposed operand) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from gqa_inputs import BF16_NAN_BITS, bf16_bits, decode_inputs, prefill_inputs, random_lens

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _f64(t):
    return oracle.bf16_bits_to_f64(bf16_bits(t))


# ---------------------------------------------------------------- bf16 widening
def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0001, 0x7F80, 0xFF80, 0x8000, 0x3C00], dtype=np.uint16)
    want = [1.0, -2.0, 3.140625, 2.0 ** -133, math.inf, -math.inf, -0.0, 2.0 ** -7]
    got = oracle.bf16_bits_to_f64(bits)
    for g, w in zip(got, want):
        assert g == w
    assert math.isnan(oracle.bf16_bits_to_f64(np.array([BF16_NAN_BITS], dtype=np.uint16))[0])


def test_bf16_widening_matches_torch_cast():
    t = torch.randn(4096, dtype=torch.float32).to(torch.bfloat16)
    got = oracle.bf16_bits_to_f64(bf16_bits(t))
    assert np.array_equal(got, t.to(torch.float64).numpy())


def test_round_to_bf16_ties_and_values():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.5, 0.0])
    want = np.array([1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.5, 0.0])
    assert np.array_equal(oracle.round_to_bf16(x), want)
    y = np.random.default_rng(0).standard_normal(10000) * 3
    assert np.array_equal(oracle.round_to_bf16(y),
                          torch.from_numpy(y).to(torch.bfloat16).to(torch.float64).numpy())


def test_default_scale_is_float32_value():
    assert oracle.default_scale(128) == float(np.float32(1 / math.sqrt(128)))
    assert abs(oracle.default_scale(128) - 0.0883883461356163) < 1e-15


def test_kv_head_map():
    assert [oracle.kv_head(h, 32, 8) for h in range(32)] == [h // 4 for h in range(32)]
    assert [oracle.kv_head(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        oracle.kv_head(0, 6, 4)


# ---------------------------------------------------------------- brute force
def _brute_prefill(q, k, v, causal, scale):
    """Pure-Python loops with math.exp: no numpy linear algebra."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    out = np.zeros(q.shape)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(S):
                keys = range(i + 1) if causal else range(S)
                logits = []
                for j in keys:
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[b, i, h, d]) * float(k[b, j, g, d])
                    logits.append(scale * acc)
                mx = max(logits)
                w = [math.exp(x - mx) for x in logits]
                tot = sum(w)
                for d in range(D):
                    out[b, i, h, d] = sum(w[n] * float(v[b, j, g, d]) for n, j in enumerate(keys)) / tot
    return out


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S,Hq,Hkv,D", [(1, 4, 2, 8), (5, 4, 2, 8), (8, 6, 3, 16), (3, 4, 1, 128)])
def test_prefill_matches_brute_force(causal, S, Hq, Hkv, D):
    q, k, v = prefill_inputs(2, S, Hq, Hkv, D, base=77 + S)
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    scale = 0.3
    got = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=causal, scale=scale)
    want = _brute_prefill(qf, kf, vf, causal, float(np.float32(scale)))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_decode_matches_brute_force():
    B, L, Hq, Hkv, D = 3, 7, 4, 2, 8
    q, kc, vc, lens = decode_inputs(B, L, Hq, Hkv, D, base=5, lens=[7, 1, 4])
    got = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), lens, scale=0.7)
    qf, kf, vf = _f64(q), _f64(kc), _f64(vc)
    s = float(np.float32(0.7))
    for b in range(B):
        n = int(lens[b])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            logits = [s * sum(qf[b, h, d] * kf[b, j, g, d] for d in range(D)) for j in range(n)]
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            for d in range(D):
                want = sum(w[j] * vf[b, j, g, d] for j in range(n)) / sum(w)
                assert abs(got[b, h, d] - want) < 1e-12


# ---------------------------------------------------------------- library routine
def _sdpa_f64(qf, kf, vf, causal, scale):
    B, S, Hq, D = qf.shape
    G = Hq // kf.shape[2]
    Q = torch.from_numpy(qf).permute(0, 2, 1, 3)
    K = torch.from_numpy(kf).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    V = torch.from_numpy(vf).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("sigma", [1.0, 16.0])
def test_prefill_matches_torch_sdpa_fp64(causal, sigma):
    q, k, v = prefill_inputs(2, 67, 8, 2, 128, base=300, sigma_qk=sigma)
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    got = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=causal, chunk=16)
    want = _sdpa_f64(qf, kf, vf, causal, oracle.default_scale(128))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)


def test_prefill_rows_and_heads_subset():
    q, k, v = prefill_inputs(1, 300, 8, 2, 128, base=400)
    full = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v))
    rows = [0, 1, 63, 64, 255, 256, 299]
    heads = [7, 0, 5]
    sub = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows=rows, heads=heads, chunk=3)
    np.testing.assert_allclose(sub, full[:, rows][:, :, heads], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- invariants and closed forms
def test_rows_of_weights_sum_to_one_and_respect_causality():
    q, k, _ = prefill_inputs(1, 33, 4, 2, 32, base=500, sigma_qk=4.0)
    P = oracle.weights(bf16_bits(q), bf16_bits(k), causal=True)
    np.testing.assert_allclose(P.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.triu(np.ones((33, 33)), 1)[None, None] * P == 0)
    assert np.all(P >= 0)
    Pn = oracle.weights(bf16_bits(q), bf16_bits(k), causal=False)
    np.testing.assert_allclose(Pn.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(Pn > 0)


def test_weights_agree_with_prefill():
    q, k, v = prefill_inputs(1, 20, 4, 2, 16, base=510)
    P = oracle.weights(bf16_bits(q), bf16_bits(k), causal=True)
    vf = _f64(v)
    out = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v))
    for h in range(4):
        np.testing.assert_allclose(out[0, :, h, :], P[0, h] @ vf[0, :, h // 2, :], rtol=0, atol=1e-12)


def test_constant_v_returns_that_constant():
    B, S, Hq, Hkv, D = 2, 40, 8, 2, 128
    q, k, _ = prefill_inputs(B, S, Hq, Hkv, D, base=600, sigma_qk=3.0)
    c = np.random.default_rng(1).integers(-8, 8, size=(B, Hkv, D)).astype(np.float64)
    vf = np.broadcast_to(c[:, None], (B, S, Hkv, D)).copy()
    for causal in (True, False):
        out = oracle.prefill(bf16_bits(q), bf16_bits(k), vf, causal=causal)
        for h in range(Hq):
            np.testing.assert_allclose(out[:, :, h, :], np.broadcast_to(c[:, None, h // 4], (B, S, D)),
                                       rtol=0, atol=1e-12)
    qd, kc, _, lens = decode_inputs(B, S, Hq, Hkv, D, base=601, lens=[40, 9])
    outd = oracle.decode(bf16_bits(qd), bf16_bits(kc), vf, lens)
    for h in range(Hq):
        np.testing.assert_allclose(outd[:, h, :], c[:, h // 4], rtol=0, atol=1e-12)


def test_single_key_returns_its_value_exactly():
    q, k, v = prefill_inputs(3, 1, 8, 2, 128, base=700, sigma_qk=16.0)
    out = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v))
    vf = _f64(v)
    for h in range(8):
        assert np.array_equal(out[:, 0, h, :], vf[:, 0, h // 4, :])
    qd, kc, vc, lens = decode_inputs(2, 50, 8, 2, 128, base=701, lens=[1, 1], poison=True)
    outd = oracle.decode(bf16_bits(qd), bf16_bits(kc), bf16_bits(vc), lens)
    vcf = _f64(vc)
    for h in range(8):
        assert np.array_equal(outd[:, h, :], vcf[:, 0, h // 4, :])


@pytest.mark.parametrize("mode", ["zero_scale", "zero_q"])
def test_uniform_weights_give_prefix_mean(mode):
    B, S, Hq, Hkv, D = 1, 37, 4, 2, 64
    q, k, v = prefill_inputs(B, S, Hq, Hkv, D, base=800)
    vf = _f64(v)
    if mode == "zero_scale":
        out = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), scale=0.0)
    else:
        out = oracle.prefill(np.zeros((B, S, Hq, D)), bf16_bits(k), bf16_bits(v))
    prefix_mean = np.cumsum(vf, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    for h in range(Hq):
        np.testing.assert_allclose(out[:, :, h, :], prefix_mean[:, :, h // 2, :], rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    B, S, Hq, Hkv, D = 2, 45, 8, 2, 128
    q, k, v = prefill_inputs(B, S, Hq, Hkv, D, base=900)
    G = Hq // Hkv
    kr = k.repeat_interleave(G, dim=2)
    vr = v.repeat_interleave(G, dim=2)
    for causal in (True, False):
        a = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=causal)
        b = oracle.prefill(bf16_bits(q), bf16_bits(kr), bf16_bits(vr), causal=causal)
        assert np.array_equal(a, b)
    # the other common head map (h % Hkv) is a different function on these inputs
    kw = k.repeat(1, 1, G, 1)
    vw = v.repeat(1, 1, G, 1)
    w = oracle.prefill(bf16_bits(q), bf16_bits(kw), bf16_bits(vw))
    assert np.max(np.abs(w - oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v)))) > 1e-2
    qd, kc, vc, lens = decode_inputs(B, 30, Hq, Hkv, D, base=901, lens=[30, 11])
    a = oracle.decode(bf16_bits(qd), bf16_bits(kc), bf16_bits(vc), lens)
    b = oracle.decode(bf16_bits(qd), bf16_bits(kc.repeat_interleave(G, dim=2)),
                      bf16_bits(vc.repeat_interleave(G, dim=2)), lens)
    assert np.array_equal(a, b)


def test_causality_later_keys_do_not_change_earlier_rows():
    B, S, Hq, Hkv, D = 1, 50, 4, 2, 64
    q, k, v = prefill_inputs(B, S, Hq, Hkv, D, base=1000)
    base_out = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v))
    cut = 23
    k2, v2 = k.clone(), v.clone()
    k2[:, cut + 1:] = (k2[:, cut + 1:].float() * -3 + 5).to(torch.bfloat16)
    v2[:, cut + 1:] = (v2[:, cut + 1:].float() * 7 - 1).to(torch.bfloat16)
    out2 = oracle.prefill(bf16_bits(q), bf16_bits(k2), bf16_bits(v2))
    assert np.array_equal(base_out[:, :cut + 1], out2[:, :cut + 1])
    assert np.max(np.abs(base_out[:, cut + 1:] - out2[:, cut + 1:])) > 1e-2


def test_key_permutation_invariance_noncausal():
    B, S, Hq, Hkv, D = 1, 64, 4, 2, 128
    q, k, v = prefill_inputs(B, S, Hq, Hkv, D, base=1100)
    perm = torch.randperm(S, generator=torch.Generator().manual_seed(3))
    a = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=False)
    b = oracle.prefill(bf16_bits(q), bf16_bits(k[:, perm]), bf16_bits(v[:, perm]), causal=False)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_decode_equals_last_row_of_causal_prefill():
    B, S, Hq, Hkv, D = 2, 70, 8, 2, 128
    q, k, v = prefill_inputs(B, S, Hq, Hkv, D, base=1200)
    pre = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows=[S - 1])
    dec = oracle.decode(bf16_bits(q[:, S - 1]), bf16_bits(k), bf16_bits(v), [S, S])
    np.testing.assert_allclose(dec, pre[:, 0], rtol=0, atol=1e-13)


def test_decode_never_reads_past_lens_and_clamps():
    B, L, Hq, Hkv, D = 4, 64, 8, 2, 128
    lens = [64, 17, 1, 0]
    q, kc, vc, ln = decode_inputs(B, L, Hq, Hkv, D, base=1300, lens=lens, poison=True)
    out = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), ln)
    assert np.all(np.isfinite(out))
    assert np.all(out[3] == 0)           # empty set -> zero row
    q2, kc2, vc2, _ = decode_inputs(B, L, Hq, Hkv, D, base=1300, lens=lens, poison=False)
    out2 = oracle.decode(bf16_bits(q2), bf16_bits(kc2), bf16_bits(vc2), ln)
    assert np.array_equal(out, out2)
    big = oracle.decode(bf16_bits(q2), bf16_bits(kc2), bf16_bits(vc2), [10 ** 6, 17, 1, -5])
    assert np.array_equal(big, out2)


@pytest.mark.parametrize("chunk", [1, 3, 7, 64, 128, 1000])
def test_split_and_lse_combine_equals_unsplit(chunk):
    B, L, Hq, Hkv, D = 3, 200, 8, 2, 128
    lens = [200, 65, 0]
    q, kc, vc, ln = decode_inputs(B, L, Hq, Hkv, D, base=1400, lens=lens, sigma_qk=8.0, poison=True)
    want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), ln)
    o_part, lse = oracle.decode_partials(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), ln, chunk)
    assert o_part.shape == (B, Hq, -(-L // chunk), D)
    assert np.all(np.isneginf(lse[2]))
    got = oracle.combine_partials(o_part, lse)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    assert np.all(got[2] == 0)


def test_combine_partials_closed_form():
    # two chunks, lse = log(1) and log(3): weights 1/4 and 3/4
    o = np.array([[[1.0, 0.0], [0.0, 2.0]]])
    lse = np.array([[0.0, math.log(3.0)]])
    np.testing.assert_allclose(oracle.combine_partials(o, lse), [[0.25, 1.5]], rtol=0, atol=1e-15)
    lse2 = np.array([[-np.inf, 5.0]])
    np.testing.assert_allclose(oracle.combine_partials(o, lse2), [[0.0, 2.0]], rtol=0, atol=0)


def test_large_logits_stay_finite_and_match_sdpa():
    q, k, v = prefill_inputs(1, 48, 4, 1, 128, base=1500, sigma_qk=16.0)
    out = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v))
    assert np.all(np.isfinite(out))
    want = _sdpa_f64(_f64(q), _f64(k), _f64(v), True, oracle.default_scale(128))
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-10)


def test_random_lens_range():
    ln = random_lens(10000, 1, 50001, seed=3)
    assert ln.dtype == torch.int32
    assert int(ln.min()) >= 1 and int(ln.max()) <= 50001


# ---------------------------------------------------------------- worked examples
def _load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_golden(), ids=lambda c: c["name"])
def test_closed_form_worked_examples(case):
    q = np.array(case["q"], dtype=np.float64)
    k = np.array(case["k"], dtype=np.float64)
    v = np.array(case["v"], dtype=np.float64)
    want = np.array(case["expected"], dtype=np.float64)
    for arr in (q, k, v):   # inputs are exact in bf16
        assert np.array_equal(oracle.round_to_bf16(arr), arr)
    if case["mode"] == "prefill":
        got = oracle.prefill(q, k, v, causal=case["causal"], scale=case["scale"])
    else:
        got = oracle.decode(q, k, v, case["lens"], scale=case["scale"])
    np.testing.assert_allclose(got, want, rtol=0, atol=case["tol"])
