"""Seeded shape fuzzing of both entry points against the oracle, and the largest batch
the decode grid accepts.

Every case draws its shape from a seeded generator, so a failure names a reproducible
case: batch, length, KV heads, group size (Hq = G * Hkv), causal flag, scale and input
spread for prefill; batch, cache capacity, per-sequence lens (including 0, negative and
past the capacity, with the unused slots NaN-poisoned) and split size for decode.
"""

import numpy as np
import pytest
import torch

import gqa_flash_attention_amd as gqa
import oracle
from gqa_inputs import D, bf16_bits, decode_inputs, prefill_inputs, randn_bf16_device
from parity_util import assert_close, dev, gpu_f64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _heads(rng):
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    return hkv * g, hkv


@pytest.mark.parametrize("case", range(12))
def test_prefill_fuzz(case):
    rng = np.random.default_rng(7100 + case)
    Hq, Hkv = _heads(rng)
    B = int(rng.integers(1, 4))
    S = int(rng.integers(1, 700))
    causal = bool(rng.integers(0, 2))
    scale = gqa.default_scale(D) if rng.integers(0, 2) else float(np.float32(rng.uniform(-0.3, 0.3)))
    sigma = float(rng.choice([1.0, 4.0]))
    _say(f"prefill fuzz {case}: B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal} scale={scale:.5f} sigma={sigma}")
    q, k, v = prefill_inputs(B, S, Hq, Hkv, base=7100 + 10 * case, sigma_qk=sigma)
    out = gqa.prefill(dev(q), dev(k), dev(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=causal, scale=scale)
    assert_close(gpu_f64(out), want, f"prefill fuzz {case}")


@pytest.mark.parametrize("case", range(10))
def test_prefill_fuzz_larger_grids(case):
    # longer prompts and batches, which reach the 8-wave and key-split forms; sampled rows
    rng = np.random.default_rng(7200 + case)
    Hq, Hkv = _heads(rng)
    B = int(rng.integers(1, 9))
    S = int(rng.integers(400, 4100))
    causal = bool(rng.integers(0, 4))   # mostly causal
    scale = gqa.default_scale(D) if rng.integers(0, 3) else float(np.float32(rng.uniform(-0.3, 0.3)))
    waves, wgs, ks = gqa.prefill_plan(B, S, Hq, Hkv)
    _say(f"prefill fuzz (larger) {case}: B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal} scale={scale:.5f} "
         f"plan {waves} waves x {wgs}, {ks} key splits")
    q, k, v = prefill_inputs(B, S, Hq, Hkv, base=7200 + 10 * case)
    out = gqa.prefill(dev(q), dev(k), dev(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = sorted(set(np.random.default_rng(case).integers(0, S, size=12).tolist()) | {0, S - 1})
    for b in sorted({0, B - 1}):
        want = oracle.prefill(bf16_bits(q[b:b + 1]), bf16_bits(k[b:b + 1]), bf16_bits(v[b:b + 1]),
                              causal=causal, scale=scale, rows=rows)
        assert_close(gpu_f64(out[b:b + 1, rows]), want, f"prefill fuzz (larger) {case}, batch element {b}")


@pytest.mark.parametrize("case", range(12))
def test_decode_fuzz(case):
    rng = np.random.default_rng(7300 + case)
    Hq, Hkv = _heads(rng)
    B = int(rng.integers(1, 10))
    L = int(rng.integers(1, 3000))
    lens = rng.integers(-2, L + 6, size=B)
    lens[rng.integers(0, B)] = 0 if rng.integers(0, 2) else L
    chunk = None if rng.integers(0, 2) else 64 * int(rng.integers(1, 17))
    _say(f"decode fuzz {case}: B={B} L={L} Hq={Hq} Hkv={Hkv} lens={lens.tolist()} chunk={chunk}")
    q, kc, vc, ln = decode_inputs(B, L, Hq, Hkv, base=7300 + 10 * case, lens=lens.astype(np.int32), poison=True)
    out = gqa.decode(dev(q), dev(kc), dev(vc), dev(ln), chunk=chunk)
    torch.cuda.synchronize()
    want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), ln)
    assert_close(gpu_f64(out), want, f"decode fuzz {case}")


def test_decode_largest_batch():
    B, L = 65535, 64
    _say(f"decode B={B} (the largest grid z) L={L}: sampled sequences")
    d = torch.device("cuda:0")
    kc = randn_bf16_device((B, L, 8, D), 7501, d)
    vc = randn_bf16_device((B, L, 8, D), 7502, d)
    q = randn_bf16_device((B, 32, D), 7500, d)
    lens_h = np.random.default_rng(7503).integers(0, L + 1, size=B).astype(np.int32)
    lens_h[[0, B - 1]] = [L, 1]
    out = gqa.decode(q, kc, vc, torch.from_numpy(lens_h).to(d))
    torch.cuda.synchronize()
    for b in [0, 1, 2, 4095, 4096, 32767, 65533, B - 1]:
        want = oracle.decode(bf16_bits(q[b:b + 1]), bf16_bits(kc[b:b + 1]), bf16_bits(vc[b:b + 1]), lens_h[b:b + 1])
        assert_close(gpu_f64(out[b:b + 1]), want, f"decode B={B}, sequence {b} (lens {lens_h[b]})")
    del kc, vc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,L", [(32, 16384), (16, 32768), (8, 65536), (64, 4096)])
def test_decode_batched_full_length_sampled_sequences(B, L):
    """The batched decodes bench.py --sweep times (same shapes, same device generator and
    seeds as its first cache copy): every sequence at the full cache length, sampled
    sequences against the oracle."""
    from gqa_inputs import seed_base
    _say(f"decode batched B={B} L={L}, plan {gqa.decode_plan(B, L, 32, 8)}: sampled sequences")
    d = torch.device("cuda:0")
    q = randn_bf16_device((B, 32, D), seed_base(4, 4), d)
    kc = randn_bf16_device((B, L, 8, D), seed_base(4, 4) + 10, d)
    vc = randn_bf16_device((B, L, 8, D), seed_base(4, 4) + 30, d)
    lens = torch.full((B,), L, dtype=torch.int32, device=d)
    out = gqa.decode(q, kc, vc, lens)
    torch.cuda.synchronize()
    for b in sorted({0, 1, B // 2, B - 1}):
        want = oracle.decode(bf16_bits(q[b:b + 1]), bf16_bits(kc[b:b + 1]), bf16_bits(vc[b:b + 1]),
                             np.array([L], dtype=np.int32))
        assert_close(gpu_f64(out[b:b + 1]), want, f"decode B={B} L={L}, sequence {b}")
    del kc, vc
    torch.cuda.empty_cache()
