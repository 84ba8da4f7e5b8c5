"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on an MI355X.

Inputs come from the seeded generator shared with the oracle; the oracle sees the
same bf16 bits. Workloads (chowfi/kernels README, "Result"): GQA 32 query heads /
8 KV heads / head size 128, bf16, causal prefill and KV-cache decode, plus the
large-value stress case (Q, K ~ N(0, 16^2)) and ragged sizes. Every test prints
the case it runs before launching it.
"""

import numpy as np
import pytest
import torch

import gqa_flash_attention_amd as gqa
import oracle
from gqa_inputs import HQ, HKV, D, bf16_bits, decode_inputs, prefill_inputs, random_lens, seed_base
from parity_util import assert_close, dev, gpu_f64, sample_rows

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _prefill_gpu(q, k, v, causal=True, scale=None):
    out = gqa.prefill(dev(q), dev(k), dev(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return out


def _decode_gpu(q, kc, vc, lens, scale=None, chunk=None):
    out = gqa.decode(dev(q), dev(kc), dev(vc), dev(lens), scale=scale, chunk=chunk)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------------ prefill, full compare
@pytest.mark.parametrize("S", [512, 1, 127, 3000])
def test_prefill_causal_full(S):
    fam, idx = (0, 0) if S == 512 else (4, [1, 127, 3000].index(S))
    _say(f"prefill causal B=1 S={S} full compare")
    q, k, v = prefill_inputs(1, S, base=seed_base(fam, idx))
    got = gpu_f64(_prefill_gpu(q, k, v))
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=True)
    assert_close(got, want, f"prefill S={S}")


@pytest.mark.parametrize("S", [2048, 4096])
def test_prefill_causal_2k_4k_full(S):
    _say(f"prefill causal B=1 S={S} full compare")
    q, k, v = prefill_inputs(1, S, base=seed_base(2, [2048, 4096].index(S)))
    got = gpu_f64(_prefill_gpu(q, k, v))
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=True)
    assert_close(got, want, f"prefill S={S}")


@pytest.mark.parametrize("S", [8192, 16384])
def test_prefill_causal_8k_16k_full(S):
    # the oracle needs ~5 s (8K) and ~22 s (16K) of 16 host threads for these
    _say(f"prefill causal B=1 S={S} full compare")
    q, k, v = prefill_inputs(1, S, base=seed_base(2, 2 + [8192, 16384, 32768].index(S)))
    got = gpu_f64(_prefill_gpu(q, k, v))
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=True)
    assert_close(got, want, f"prefill S={S}")


@pytest.mark.parametrize("S", [32768])
def test_prefill_causal_full_size_sampled_rows(S):
    _say(f"prefill causal B=1 S={S}, sampled rows x all heads")
    q, k, v = prefill_inputs(1, S, base=seed_base(2, 2 + [8192, 16384, 32768].index(S)))
    out = _prefill_gpu(q, k, v)
    rows = sorted(set(sample_rows(S, extra=64, seed=S)) | set(range(S - 128, S)))
    got = gpu_f64(out[:, rows])
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=True, rows=rows)
    assert_close(got, want, f"prefill S={S} sampled")


def test_prefill_stress_large_logits_full():
    _say("prefill stress S=4096, Q,K ~ N(0,16^2), full compare")
    q, k, v = prefill_inputs(1, 4096, base=seed_base(3, 0), sigma_qk=16.0)
    got = gpu_f64(_prefill_gpu(q, k, v))
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=True)
    assert_close(got, want, "prefill stress")


@pytest.mark.parametrize("S", [1, 64, 200, 333])
def test_prefill_noncausal(S):
    _say(f"prefill non-causal B=1 S={S}")
    q, k, v = prefill_inputs(1, S, base=5000 + S)
    got = gpu_f64(_prefill_gpu(q, k, v, causal=False))
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=False)
    assert_close(got, want, f"prefill non-causal S={S}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (64, 8), (12, 4), (6, 2), (32, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_other_group_sizes_and_batch(Hq, Hkv, causal):
    B, S = 2, 161
    _say(f"prefill B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal}")
    q, k, v = prefill_inputs(B, S, Hq, Hkv, D, base=6000 + Hq + Hkv)
    got = gpu_f64(_prefill_gpu(q, k, v, causal=causal))
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=causal)
    assert_close(got, want, f"prefill Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("scale", [0.0, -0.0883883461356163, 0.5, 1e-3])
def test_prefill_other_scales(scale):
    _say(f"prefill S=300 scale={scale}")
    q, k, v = prefill_inputs(1, 300, base=6500)
    got = gpu_f64(_prefill_gpu(q, k, v, scale=scale))
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=True, scale=scale)
    assert_close(got, want, f"prefill scale={scale}")


# ------------------------------------------------------------------ prefill, exact properties
def test_prefill_single_key_is_exact():
    _say("prefill S=1: out == V[0] bitwise")
    q, k, v = prefill_inputs(3, 1, base=7000, sigma_qk=16.0)
    out = _prefill_gpu(q, k, v)
    want = v.repeat_interleave(HQ // HKV, dim=2)
    assert torch.equal(out.cpu(), want)


def test_prefill_gqa_equals_mha_with_repeated_kv_bitwise():
    _say("prefill S=700: GQA (8 KV heads) vs MHA with repeated KV, bitwise")
    q, k, v = prefill_inputs(1, 700, base=7100)
    a = _prefill_gpu(q, k, v).cpu()
    b = _prefill_gpu(q, k.repeat_interleave(4, dim=2), v.repeat_interleave(4, dim=2)).cpu()
    assert torch.equal(a, b)


def test_prefill_causality_bitwise_and_deterministic():
    S, cut = 1000, 411
    _say(f"prefill S={S}: rows <= {cut} unchanged when later K/V change; repeat runs identical")
    q, k, v = prefill_inputs(1, S, base=7200)
    a = _prefill_gpu(q, k, v).cpu()
    a2 = _prefill_gpu(q, k, v).cpu()
    assert torch.equal(a, a2)
    k2, v2 = k.clone(), v.clone()
    k2[:, cut + 1:] = (k2[:, cut + 1:].float() * -2.5 + 1).to(torch.bfloat16)
    v2[:, cut + 1:] = (v2[:, cut + 1:].float() * 3 - 2).to(torch.bfloat16)
    b = _prefill_gpu(q, k2, v2).cpu()
    assert torch.equal(a[:, :cut + 1], b[:, :cut + 1])
    assert not torch.equal(a[:, cut + 1:], b[:, cut + 1:])


def test_prefill_constant_v_and_zero_scale_prefix_mean():
    S = 257
    _say(f"prefill S={S}: constant V; scale 0 gives the prefix mean")
    q, k, _ = prefill_inputs(1, S, base=7300, sigma_qk=4.0)
    c = torch.randint(-8, 8, (1, 1, HKV, D)).to(torch.bfloat16)
    v = c.expand(1, S, HKV, D).contiguous()
    out = gpu_f64(_prefill_gpu(q, k, v))
    want = np.broadcast_to(gpu_f64(c.repeat_interleave(4, dim=2)), out.shape)
    assert_close(out, want, "constant V")
    _, _, v = prefill_inputs(1, S, base=7301)
    out = gpu_f64(_prefill_gpu(q, k, v, scale=0.0))
    vf = oracle.bf16_bits_to_f64(bf16_bits(v))
    pm = np.cumsum(vf, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    assert_close(out, np.repeat(pm, 4, axis=2), "prefix mean")


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("L", [2048, 4096, 8192, 16384, 32768, 65536])
def test_decode_full(L):
    idx = [2048, 4096, 8192, 16384, 32768, 65536].index(L)
    _say(f"decode B=1 L={L} full compare (library split)")
    q, kc, vc, lens = decode_inputs(1, L, base=seed_base(1, idx))
    got = gpu_f64(_decode_gpu(q, kc, vc, lens))
    want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), lens)
    assert_close(got, want, f"decode L={L}")


def test_decode_stress_large_logits():
    _say("decode stress L=16384, q,K ~ N(0,16^2)")
    q, kc, vc, lens = decode_inputs(1, 16384, base=seed_base(3, 1), sigma_qk=16.0)
    got = gpu_f64(_decode_gpu(q, kc, vc, lens))
    want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), lens)
    assert_close(got, want, "decode stress")


def test_decode_ragged_batch_nan_poisoned():
    B, L = 16, 50001
    _say(f"decode ragged B={B} L={L}, lens ~ U[1, 50001], slots >= lens hold NaN")
    lens = random_lens(B, 1, L, seed=seed_base(4, 3) + 3)
    q, kc, vc, lens = decode_inputs(B, L, base=seed_base(4, 3), lens=lens, poison=True)
    got = gpu_f64(_decode_gpu(q, kc, vc, lens))
    want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), lens)
    assert_close(got, want, "decode ragged")


@pytest.mark.parametrize("L,chunk", [(256, 256), (128, 64), (192, 64), (400, 64), (1000, 128),
                                     (1000, 192), (5000, 256), (64, 64), (65, 64), (3000, 512),
                                     (3000, 3008), (5000, 1024), (20000, 4096), (777, 832)])
def test_decode_forced_splits(L, chunk):
    nsplit = -(-L // chunk)
    _say(f"decode B=2 L={L} chunk={chunk} (nsplit={nsplit}), ragged lens, NaN padding")
    q, kc, vc, lens = decode_inputs(2, L, base=8000 + L, lens=[L, max(1, L // 3)], poison=True)
    got = gpu_f64(_decode_gpu(q, kc, vc, lens, chunk=chunk))
    want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), lens)
    assert_close(got, want, f"decode chunk={chunk}")


def test_decode_split_counts_agree():
    L = 3000
    _say(f"decode L={L}: every split size matches the oracle and the others")
    q, kc, vc, lens = decode_inputs(1, L, base=8100)
    want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), lens)
    outs = {}
    for chunk in (64, 128, 192, 256, 640, 1024, 3008):
        outs[chunk] = gpu_f64(_decode_gpu(q, kc, vc, lens, chunk=chunk))
        assert_close(outs[chunk], want, f"chunk={chunk}")
    for c in (128, 192, 256, 640, 1024, 3008):
        assert np.max(np.abs(outs[c] - outs[64])) <= 2e-2


def test_decode_partials_match_oracle_split():
    L, chunk = 1100, 128
    _say(f"decode partials L={L} chunk={chunk} vs oracle split (lse in log2 units)")
    lens = [L, 300, 1]
    q, kc, vc, ln = decode_inputs(3, L, base=8200, lens=lens, poison=True)
    o_part, lse, ws = gqa.decode_partials(dev(q), dev(kc), dev(vc), dev(ln), chunk)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_partials(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), ln, chunk)
    lse_g = lse.cpu().double().numpy()
    lse_ref2 = lse_ref / np.log(2.0)
    empty = np.isneginf(lse_ref2)
    assert np.array_equal(np.isneginf(lse_g), empty)
    assert np.max(np.abs(lse_g[~empty] - lse_ref2[~empty])) < 2e-2
    og = o_part.cpu().double().numpy()
    valid = ~empty
    assert np.max(np.abs(og[valid] - o_ref[valid])) < 2e-2
    assert np.mean(np.abs(og[valid] - o_ref[valid])) < 2e-3
    out = gqa.decode_combine(ws, 3, HQ, -(-L // chunk))
    torch.cuda.synchronize()
    want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), ln)
    assert_close(gpu_f64(out), want, "combine of GPU partials")


def test_decode_single_key_exact_and_empty_and_clamped():
    B, L = 4, 300
    _say("decode lens = [1, 0, L+50 (clamped), -3]: exact V row, zero rows, clamp")
    q, kc, vc, _ = decode_inputs(B, L, base=8300, sigma_qk=16.0)
    lens = torch.tensor([1, 0, L + 50, -3], dtype=torch.int32)
    out = _decode_gpu(q, kc, vc, lens).cpu()
    assert torch.equal(out[0], vc[0, 0].repeat_interleave(4, dim=0))
    assert torch.all(out[1].float() == 0) and torch.all(out[3].float() == 0)
    want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), [1, 0, L, 0])
    assert_close(gpu_f64(out), want, "decode lens edge cases")


def test_decode_single_split_with_empty_sequence():
    _say("decode B=3 L=500 one split (chunk 512), lens = [500, 0, 37]")
    q, kc, vc, lens = decode_inputs(3, 500, base=8350, lens=[500, 0, 37], poison=True)
    out = _decode_gpu(q, kc, vc, lens, chunk=512)
    assert torch.all(out[1].float().cpu() == 0)
    want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), lens)
    assert_close(gpu_f64(out), want, "decode one split")


def test_decode_workspace_reused_across_calls():
    _say("decode with one caller workspace, calls of two shapes in a row: the merge counters return to zero")
    q, kc, vc, lens = decode_inputs(2, 4000, base=8360, lens=[4000, 2500], poison=True)
    ws = gqa.decode_workspace(2, 4000, HQ, HKV, D, 256, device="cuda:0")
    ncnt = max(4096, 2 * HQ) * 4
    out1 = gqa.decode(dev(q), dev(kc), dev(vc), dev(lens), chunk=256, workspace=ws)
    torch.cuda.synchronize()
    assert bool((ws[:ncnt] == 0).all())
    q2, kc2, vc2, lens2 = decode_inputs(1, 1500, base=8361, lens=[1400], poison=True)
    out2 = gqa.decode(dev(q2), dev(kc2), dev(vc2), dev(lens2), chunk=256, workspace=ws)
    out3 = gqa.decode(dev(q), dev(kc), dev(vc), dev(lens), chunk=256, workspace=ws)
    torch.cuda.synchronize()
    assert bool((ws[:ncnt] == 0).all())
    assert_close(gpu_f64(out1), oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), lens), "call 1")
    assert_close(gpu_f64(out2), oracle.decode(bf16_bits(q2), bf16_bits(kc2), bf16_bits(vc2), lens2), "call 2")
    assert torch.equal(out1.cpu(), out3.cpu())


def test_decode_large_batch_uses_more_than_the_minimum_counters():
    # B * Hq = 4352 merge counters, past the 4096 every workspace holds at least; the
    # library's workspace of this stream grows and its new counters are cleared
    B, L = 136, 320
    _say(f"decode B={B} L={L} on the library workspace: {B * HQ} merge counters")
    lens = random_lens(B, 1, L, seed=8390)
    q, kc, vc, lens = decode_inputs(B, L, base=8391, lens=lens, poison=True)
    first = _decode_gpu(q, kc, vc, lens)
    again = _decode_gpu(q, kc, vc, lens)
    assert torch.equal(first, again)
    rows = [0, 1, 67, B - 2, B - 1]
    got = gpu_f64(first[rows])
    want = oracle.decode(bf16_bits(q[rows]), bf16_bits(kc[rows]), bf16_bits(vc[rows]), lens[rows])
    assert_close(got, want, f"decode B={B}")


def test_decode_other_group_sizes_and_scales():
    for (Hq, Hkv, scale) in [(8, 8, None), (64, 8, None), (40, 2, None), (32, 8, 0.0), (32, 8, -0.3)]:
        _say(f"decode B=2 L=700 Hq={Hq} Hkv={Hkv} scale={scale}")
        q, kc, vc, lens = decode_inputs(2, 700, Hq, Hkv, D, base=8400 + Hq, lens=[700, 123], poison=True)
        got = gpu_f64(_decode_gpu(q, kc, vc, lens, scale=scale))
        want = oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), lens, scale=scale)
        assert_close(got, want, f"decode Hq={Hq} Hkv={Hkv}")


def test_decode_deterministic_and_equals_last_prefill_row():
    S = 777
    _say(f"decode L={S} twice (bitwise) and against the last causal prefill row")
    q, k, v = prefill_inputs(1, S, base=8500)
    qd = q[:, S - 1].contiguous()
    lens = torch.tensor([S], dtype=torch.int32)
    a = _decode_gpu(qd, k, v, lens).cpu()
    b = _decode_gpu(qd, k, v, lens).cpu()
    assert torch.equal(a, b)
    p = _prefill_gpu(q, k, v).cpu()[:, S - 1]
    assert np.max(np.abs(gpu_f64(a) - gpu_f64(p))) <= 2e-2


def test_invalid_arguments_on_gpu_raise_cleanly():
    _say("error paths with real device tensors")
    q, k, v = prefill_inputs(1, 64, base=8600)
    qd, kd, vd = dev(q), dev(k), dev(v)
    with pytest.raises(gqa.GqaAttnError):
        gqa.prefill(qd[..., :64].contiguous(), kd[..., :64].contiguous(), vd[..., :64].contiguous())
    flat = torch.empty(qd.numel() + 8, dtype=torch.bfloat16, device="cuda:0")
    mis = flat[1:1 + qd.numel()].view_as(qd)
    with pytest.raises(gqa.GqaAttnError):
        gqa.prefill(mis, kd, vd)
    torch.cuda.synchronize()


def test_workspace_and_output_checks_in_the_binding():
    _say("decode workspace on the host, of the wrong dtype or too small; combine output of the wrong shape")
    q, kc, vc, lens = [dev(t) for t in decode_inputs(1, 300, base=8700)]
    need = gqa.decode_workspace_bytes(1, 300, 32, 8, 128)
    with pytest.raises(ValueError):
        gqa.decode(q, kc, vc, lens, workspace=torch.zeros(need, dtype=torch.uint8))        # host memory
    with pytest.raises(ValueError):
        gqa.decode(q, kc, vc, lens, workspace=torch.zeros(need // 4 + 1, dtype=torch.int32, device="cuda:0"))
    with pytest.raises(gqa.GqaAttnError):
        gqa.decode(q, kc, vc, lens, workspace=torch.zeros(64, dtype=torch.uint8, device="cuda:0"))
    o_part, lse, ws = gqa.decode_partials(q, kc, vc, lens, 128)
    with pytest.raises(ValueError):
        gqa.decode_combine(ws, 1, 32, 3, out=torch.empty((1, 32, 64), dtype=torch.bfloat16, device="cuda:0"))
    with pytest.raises(ValueError):
        gqa.decode_combine(ws.cpu(), 1, 32, 3)
    good = gqa.decode_combine(ws, 1, 32, 3)
    torch.cuda.synchronize()
    assert torch.isfinite(good.float()).all()
