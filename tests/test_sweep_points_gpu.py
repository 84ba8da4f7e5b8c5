"""Parity of every point of the decode split-size sweep (bench.py --sweep-chunks):
the same seeded inputs the bench uses, each runnable chunk, against the oracle."""

import pytest
import torch

import bench
import gqa_flash_attention_amd as gqa
import oracle
from gqa_inputs import bf16_bits
from parity_util import assert_close, gpu_f64

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
