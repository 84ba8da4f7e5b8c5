"""Seeded synthetic inputs for GQA attention, shared by the tests and the benchmark.

This module only draws random numbers and lays them out. It holds none of the
attention arithmetic, so the oracle and the HIP path can both take their
inputs from here without sharing any of the method.

Recipe (every tensor is generated on the CPU, so both sides see the same
bits):
- draw float32 N(0, 1) with ``torch.Generator('cpu').manual_seed(seed)``;
- multiply by sigma;
- round to bf16 (torch's round-to-nearest-even).

Seeds: for workload family c and size index i, base = 1000*c + 10*i, and
q, k, v, lens take base+0, base+1, base+2 and base+3.

The workload is the attention step of a Llama-3-8B-size model: 32 query heads,
8 KV heads, head size 128, bf16 (chowfi/kernels README, "Result", settings
line). No dataset is involved; random activations of that shape stand in for
the page's benchmark inputs.
"""

from __future__ import annotations

import numpy as np
import torch

HQ, HKV, D = 32, 8, 128
BF16_NAN_BITS = 0x7FC0   # a quiet bf16 NaN, used to poison unused cache slots

__all__ = [
    "HQ", "HKV", "D", "BF16_NAN_BITS", "seed_base", "randn_bf16", "randn_bf16_device",
    "prefill_inputs", "decode_inputs", "random_lens", "bf16_bits",
]


def seed_base(family: int, size_index: int = 0) -> int:
    return 1000 * int(family) + 10 * int(size_index)


def randn_bf16(shape, seed: int, sigma: float = 1.0) -> torch.Tensor:
    """CPU bf16 tensor of N(0, sigma^2) values drawn from ``seed``."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if sigma != 1.0:
        x = x * float(sigma)
    return x.to(torch.bfloat16)


def randn_bf16_device(shape, seed: int, device, sigma: float = 1.0) -> torch.Tensor:
    """bf16 N(0, sigma^2) values drawn on the device from ``seed`` (for inputs too large to
    draw on the host). The same seed and device give the same bits; copy a slice to the
    host to hand it to a CPU reference."""
    g = torch.Generator(device=device).manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if sigma != 1.0:
        x.mul_(float(sigma))
    return x.to(torch.bfloat16)


def prefill_inputs(B: int, S: int, Hq: int = HQ, Hkv: int = HKV, Dh: int = D,
                   base: int = 0, sigma_qk: float = 1.0, sigma_v: float = 1.0):
    """(q [B,S,Hq,D], k [B,S,Hkv,D], v [B,S,Hkv,D]) as CPU bf16 tensors."""
    q = randn_bf16((B, S, Hq, Dh), base + 0, sigma_qk)
    k = randn_bf16((B, S, Hkv, Dh), base + 1, sigma_qk)
    v = randn_bf16((B, S, Hkv, Dh), base + 2, sigma_v)
    return q, k, v


def random_lens(B: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """int32 [B] drawn uniformly from [lo, hi] inclusive."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    return torch.randint(int(lo), int(hi) + 1, (B,), generator=g, dtype=torch.int32)


def decode_inputs(B: int, L: int, Hq: int = HQ, Hkv: int = HKV, Dh: int = D,
                  base: int = 0, lens=None, sigma_qk: float = 1.0, sigma_v: float = 1.0,
                  poison: bool = False):
    """(q [B,Hq,D], kcache [B,L,Hkv,D], vcache [B,L,Hkv,D], lens int32 [B]) on the CPU.

    lens defaults to L for every sequence. With ``poison``, every cache slot at
    or past lens[b] holds a bf16 NaN, so a kernel that reads one shows it.
    """
    q = randn_bf16((B, Hq, Dh), base + 0, sigma_qk)
    kc = randn_bf16((B, L, Hkv, Dh), base + 1, sigma_qk)
    vc = randn_bf16((B, L, Hkv, Dh), base + 2, sigma_v)
    if lens is None:
        lens = torch.full((B,), L, dtype=torch.int32)
    else:
        lens = torch.as_tensor(lens, dtype=torch.int32).reshape(B).clone()
    if poison:
        nan = torch.tensor(BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16)
        for b in range(B):
            n = int(min(max(int(lens[b]), 0), L))
            if n < L:
                kc[b, n:] = nan
                vc[b, n:] = nan
    return q, kc, vc, lens


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a bf16 tensor (moved to the CPU if needed)."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bf16 tensor")
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
