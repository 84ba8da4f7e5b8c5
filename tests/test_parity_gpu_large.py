"""Hardened parity on the GPU: sizes past 2^31 elements, layout errors, key order.

- Offsets past 2^31 elements: a prefill whose q/out hold 2.7e9 elements (B=80,
  S=8192) and a decode whose caches hold 2^32 elements each (B=2, L=2^21); outputs
  whose inputs sit past 2^31 elements (and past 2^32 bytes) are checked against the
  oracle, so 32-bit index arithmetic anywhere on the path would show.
- Non-contiguous or mis-typed tensors are rejected before anything runs.
- Key order: with causal=False, permuting the keys (K and V rows together) changes
  only the summation order, so the GPU result must stay within the same tolerance of
  the oracle and close to the unpermuted GPU result (the reference as a band, as the
  metakernel page describes for reordered reductions).
"""

import numpy as np
import pytest
import torch

import gqa_flash_attention_amd as gqa
import oracle
from gqa_inputs import HKV, HQ, D, bf16_bits, decode_inputs, prefill_inputs, randn_bf16_device
from parity_util import assert_close, dev, gpu_f64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def test_prefill_past_2pow31_elements():
    B, S = 80, 8192
    n = B * S * HQ * D
    _say(f"prefill B={B} S={S}: q/out hold {n} elements ({n * 2} bytes); sampled rows of the first and last batch element")
    d = torch.device("cuda:0")
    q = randn_bf16_device((B, S, HQ, D), 9100, d)
    k = randn_bf16_device((B, S, HKV, D), 9101, d)
    v = randn_bf16_device((B, S, HKV, D), 9102, d)
    out = gqa.prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 4095, 4096, S - 2, S - 1]
    for b in (0, B - 1):
        got = gpu_f64(out[b:b + 1, rows])
        want = oracle.prefill(bf16_bits(q[b:b + 1]), bf16_bits(k[b:b + 1]), bf16_bits(v[b:b + 1]),
                              causal=True, rows=rows)
        assert_close(got, want, f"prefill past 2^31 elements, batch element {b}")
    del q, k, v, out
    torch.cuda.empty_cache()


def test_decode_cache_past_2pow31_elements():
    """Caches of 2^32 elements each. A split's partial result depends only on its own
    slots, so sampled splits are checked against the oracle one by one: the first split,
    the split at 2^30 elements into sequence 0, the first split of sequence 1 (2^31
    elements in) and the ragged last split of sequence 1 (near 2^32 elements)."""
    B, L, chunk = 2, 1 << 21, 4096
    _say(f"decode B={B} L={L} chunk={chunk}: each cache holds {B * L * HKV * D} elements; sampled splits")
    d = torch.device("cuda:0")
    kc = randn_bf16_device((B, L, HKV, D), 9201, d)
    vc = randn_bf16_device((B, L, HKV, D), 9202, d)
    q = randn_bf16_device((B, HQ, D), 9200, d)
    lens_h = [L, L - 3]
    lens = torch.tensor(lens_h, dtype=torch.int32, device=d)
    o_part, lse, ws = gqa.decode_partials(q, kc, vc, lens, chunk)
    nsplit = L // chunk
    torch.cuda.synchronize()
    qh = bf16_bits(q)
    for b, c in [(0, 0), (0, nsplit // 2), (1, 0), (1, nsplit - 1)]:
        j0, j1 = c * chunk, min((c + 1) * chunk, lens_h[b])
        o_ref, lse_ref = oracle.decode_partials(qh[b:b + 1], bf16_bits(kc[b:b + 1, j0:j1]),
                                                bf16_bits(vc[b:b + 1, j0:j1]), [j1 - j0], j1 - j0)
        og = o_part[b, :, c].cpu().double().numpy()
        assert np.max(np.abs(og - o_ref[0, :, 0])) < 2e-2, (b, c)
        assert np.mean(np.abs(og - o_ref[0, :, 0])) < 2e-3, (b, c)
        lg = lse[b, :, c].cpu().double().numpy()
        assert np.max(np.abs(lg - lse_ref[0, :, 0] / np.log(2.0))) < 2e-2, (b, c)
    # the fused single-launch decode assigns keys to splits its own way (strided tiles);
    # it must agree with the stand-alone merge of the chunk results up to summation
    # order: the outputs here are ~1e-3 in size, so 1e-4 is a few of their bf16 ulps
    split_out = gqa.decode_combine(ws, B, HQ, nsplit)
    fused = gqa.decode(q, kc, vc, lens, chunk=chunk)
    auto = gqa.decode(q, kc, vc, lens)
    torch.cuda.synchronize()
    a, f, u = split_out.double(), fused.double(), auto.double()
    assert torch.all(torch.isfinite(f)) and float(a.abs().max()) > 0
    assert float((a - f).abs().max()) <= 1e-4
    assert float((a - u).abs().max()) <= 1e-4
    del kc, vc, ws
    torch.cuda.empty_cache()


def test_layout_and_dtype_errors():
    _say("non-contiguous, wrong dtype, wrong device and mismatched shapes are rejected")
    q, k, v = prefill_inputs(1, 64, base=9300)
    qd, kd, vd = dev(q), dev(k), dev(v)
    with pytest.raises(ValueError):
        gqa.prefill(qd.transpose(1, 2).contiguous().transpose(1, 2), kd, vd)   # same shape, not contiguous
    with pytest.raises(TypeError):
        gqa.prefill(qd.float(), kd, vd)
    with pytest.raises(ValueError):
        gqa.prefill(q, k, v)                                                    # host tensors
    with pytest.raises(ValueError):
        gqa.prefill(qd, kd[:, :32].contiguous(), vd)
    qd2, kc, vc, lens = decode_inputs(1, 100, base=9301)
    with pytest.raises(ValueError):
        gqa.decode(dev(qd2), dev(kc), dev(vc), dev(lens).to(torch.int64))
    with pytest.raises(ValueError):
        gqa.decode(dev(qd2), dev(kc)[:, ::2].contiguous(), dev(vc), dev(lens))


@pytest.mark.parametrize("S", [130, 1000])
def test_key_permutation_band(S):
    _say(f"prefill non-causal S={S}: keys permuted vs not, both against the oracle")
    q, k, v = prefill_inputs(1, S, base=9400 + S)
    perm = torch.randperm(S, generator=torch.Generator().manual_seed(S))
    a = gpu_f64(gqa.prefill(dev(q), dev(k), dev(v), causal=False))
    b = gpu_f64(gqa.prefill(dev(q), dev(k[:, perm]), dev(v[:, perm]), causal=False))
    torch.cuda.synchronize()
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=False)
    assert_close(a, want, "original key order")
    assert_close(b, want, "permuted key order")
    # the two GPU results differ only by summation order: within two bf16 steps
    assert np.max(np.abs(a - b)) <= 2 * np.max(np.abs(oracle.round_to_bf16(want) - want)) + 1e-2
