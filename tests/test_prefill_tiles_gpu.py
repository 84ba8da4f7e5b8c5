"""Prefill parity of every tile shape of gqa_attn_prefill_tiles (32- and 128-key tiles,
64 rows per wave) beyond the sweep's own sizes: short and ragged prompts, other group
sizes, batches, causal and not, a negative scale (the other arm of the scale folding) and
the large-value stress inputs, each a full compare against the oracle."""

import pytest
import torch

import gqa_flash_attention_amd as gqa
import oracle
from gqa_inputs import D, bf16_bits, prefill_inputs
from parity_util import assert_close, dev, gpu_f64

pytestmark = pytest.mark.gpu

SHAPES = [t for t in gqa.PREFILL_TILES if t not in ((32, 64, 4), (32, 64, 8))]

# (B, S, Hq, Hkv, causal, scale, sigma_qk)
CASES = [
    (1, 1, 32, 8, True, None, 1.0),
    (1, 100, 32, 8, True, None, 1.0),
    (2, 333, 32, 8, False, None, 1.0),
    (1, 777, 8, 8, True, None, 1.0),          # G = 1: a wave's two units are two row blocks
    (2, 300, 48, 8, True, -0.0883883461356163, 1.0),   # G = 6
    (1, 1100, 32, 8, True, None, 16.0),       # large logits
    (3, 161, 32, 4, True, 0.0, 1.0),          # scale 0: prefix means
]


@pytest.mark.parametrize("tiles", SHAPES)
@pytest.mark.parametrize("B,S,Hq,Hkv,causal,scale,sigma", CASES)
def test_prefill_tile_shape_matches_oracle(tiles, B, S, Hq, Hkv, causal, scale, sigma):
    print(f"[case] prefill tiles={tiles} B={B} S={S} Hq={Hq} Hkv={Hkv} causal={causal} scale={scale} "
          f"sigma={sigma}", flush=True)
    q, k, v = prefill_inputs(B, S, Hq, Hkv, D, base=13000 + B + S + Hq, sigma_qk=sigma)
    out = gqa.prefill(dev(q), dev(k), dev(v), causal=causal, scale=scale, tiles=tiles)
    torch.cuda.synchronize()
    want = oracle.prefill(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=causal, scale=scale)
    assert_close(gpu_f64(out), want, f"tiles={tiles} B={B} S={S} Hq={Hq} Hkv={Hkv}")
