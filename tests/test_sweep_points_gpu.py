"""Parity of every point of the three sweeps, on the same seeded inputs the bench uses:
each runnable chunk of the decode split-size sweep (bench.py --sweep-chunks), each
workgroup form of the prefill form sweep (bench.py --sweep-forms) and each tile shape of
the prefill tile sweep (bench.py --sweep-tiles), against the oracle."""

import pytest
import torch

import bench
import gqa_flash_attention_amd as gqa
import oracle
from gqa_inputs import bf16_bits
from parity_util import assert_close, gpu_f64, sample_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("L", bench.SWEEP_CHUNK_L)
def test_every_sweep_chunk_matches_oracle(L):
    d = torch.device("cuda:0")
    default, run, skip = bench.chunk_candidates(L)
    print(f"[case] sweep points L={L}: default {default}, run {run}, not run {[c for c, _ in skip]}", flush=True)
    qd, kc, vc, lens = bench.make_inputs(64, L, d)[3:]
    want = oracle.decode(bf16_bits(qd), bf16_bits(kc), bf16_bits(vc), lens.cpu())
    for c in run:
        out = gqa.decode(qd, kc, vc, lens, chunk=c)
        torch.cuda.synchronize()
        assert_close(gpu_f64(out), want, f"decode L={L} chunk={c}")


@pytest.mark.parametrize("S", bench.SWEEP_FORM_S)
def test_every_sweep_form_matches_oracle(S):
    d = torch.device("cuda:0")
    print(f"[case] sweep points prefill S={S}: forms {gqa.PREFILL_FORMS}, plan {gqa.prefill_plan(1, S, 32, 8)}",
          flush=True)
    q, k, v = bench.make_inputs(S, 64, d)[:3]
    rows = sample_rows(S, seed=S)
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=True, rows=rows)
    outs = {}
    for fm in gqa.PREFILL_FORMS:
        outs[fm] = gqa.prefill(q, k, v, form=fm)
        torch.cuda.synchronize()
        assert_close(gpu_f64(outs[fm][:, rows]), want, f"prefill S={S} form={fm}")
    # the one-wave-per-unit forms give each wave the same rows and operation order
    assert torch.equal(outs[(4, 1)], outs[(8, 1)])
    assert torch.equal(gqa.prefill(q, k, v), outs[gqa.prefill_plan(1, S, 32, 8)[::2]])


@pytest.mark.parametrize("S", bench.SWEEP_TILE_S)
def test_every_sweep_tile_shape_matches_oracle(S):
    d = torch.device("cuda:0")
    print(f"[case] sweep points prefill S={S}: tile shapes {gqa.PREFILL_TILES}", flush=True)
    q, k, v = bench.make_inputs(S, 64, d)[:3]
    rows = sorted(set(sample_rows(S, seed=S)) | set(range(max(0, S - 64), S)))
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=True, rows=rows)
    outs = {}
    for tl in gqa.PREFILL_TILES:
        outs[tl] = gqa.prefill(q, k, v, tiles=tl)
        torch.cuda.synchronize()
        assert_close(gpu_f64(outs[tl][:, rows]), want, f"prefill S={S} tiles={tl}")
    # the first two are the library's own forms, bit for bit
    assert torch.equal(outs[(32, 64, 4)], gqa.prefill(q, k, v, form=(4, 1)))
    assert torch.equal(outs[(32, 64, 8)], gqa.prefill(q, k, v, form=(8, 1)))
