"""Plain, slow, float64 CPU reference for GQA attention forward.

TEST INFRASTRUCTURE ONLY. This is the oracle the HIP kernels are checked
against. Product code never imports it; it imports nothing from the product.

Source: the README of the ``chowfi/kernels`` repository ("Autoresearch made a
custom GPU kernel for consumer hardware faster than Flash Attention 2").
- Intro paragraph: the operation is the attention step of a Llama-3-8B-size
  model, grouped-query attention (GQA), forward pass only.
- "Result", settings line: bf16, batch 1, 32 query heads, 8 KV heads, head
  size 128.
- "Result", the two mode bullets: prefill processes the full prompt with a
  causal mask; decode produces one token from a KV cache of a given length.
- "What helped most", item 2: each group of 4 query heads shares one KV head.
- "What helped most", item 1: decode may split the KV cache into chunks and
  combine the results. ``decode_partials``/``combine_partials`` write that
  split out so it can be checked against the unsplit definition.

The page never writes the formula. It benchmarks against FlashAttention-2 and
PyTorch SDPA as the same function ("Result", the SDPA sentence), so the
definition taken is standard scaled-dot-product softmax attention:

    x[i, j]   = scale * sum_d Q[b, i, h, d] * K[b, j, g(h), d]     for j in vis(i)
    out[i, :] = sum_{j in vis(i)} softmax_j(x[i, :]) * V[b, j, g(h), :]

Readings taken where the page is silent:
- g(h) = h // (Hq // Hkv): contiguous groups, i.e. K/V heads repeated with
  repeat_interleave.
- Layout is BSHD: q/out [B, S, Hq, D], k/v [B, S, Hkv, D]. Decode takes q/out
  [B, Hq, D] and caches [B, L, Hkv, D], where L is the capacity.
- Causal: query i sees keys 0..i, diagonal included. Non-causal: all S keys.
- Decode: the query sees cache slots 0..lens[b]-1. lens is clamped to [0, L],
  and an empty set gives a zero row.
- scale is the float32 value the caller passes (default float32(1/sqrt(D))),
  promoted exactly to float64.
- Inputs are bf16 bit patterns, widened exactly to float64 (bf16 is a subset
  of float32, which is a subset of float64).

Arithmetic: float64 throughout. The softmax is the exact two-pass form (max,
exp, sum, divide) over the visible keys only. There is no online softmax, no
tiling of the key axis and no split, except in the two split helpers, which
exist to be checked against this definition.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "round_to_bf16",
    "default_scale",
    "kv_head",
    "prefill",
    "decode",
    "weights",
    "decode_partials",
    "combine_partials",
]


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64.

    A bf16 value is the top 16 bits of a float32, so shifting its bits up by
    16 gives that float32 exactly. Widening float32 to float64 is exact too.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        b = b.astype(np.int64).astype(np.uint16)
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    This is used only to measure the bf16 output-rounding floor that any bf16
    result carries. The float64 value is first rounded to float32 (RNE), then
    to bf16 (RNE on the low 16 bits). The double rounding can differ from a
    single rounding only on exact float32 ties, which are far below the
    tolerances this is compared with.
    """
    f32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = rounded.astype(np.uint32).view(np.float32).astype(np.float64)
    nan = np.isnan(f32)
    out[nan] = np.nan
    return out


def default_scale(D: int) -> float:
    """float32(1/sqrt(D)) promoted to float64: the scale a caller gets by default."""
    return float(np.float32(1.0) / np.sqrt(np.float32(D)))


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """KV head that query head h reads: g(h) = h // (Hq // Hkv)."""
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64, copy=False)


def _softmax_rows(x: np.ndarray) -> np.ndarray:
    """Exact two-pass softmax over the last axis, float64. The rows must not be empty."""
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def prefill(q, k, v, causal: bool = True, scale: float | None = None,
            rows=None, heads=None, chunk: int = 256) -> np.ndarray:
    """Attention over a full prompt.

    q: [B, S, Hq, D]; k, v: [B, S, Hkv, D]. Either bf16 bits (uint16) or floats.
    rows: optional sequence of query positions to evaluate (default: all S).
    heads: optional sequence of query heads to evaluate (default: all Hq).
    Returns float64 [B, len(rows), len(heads), D].

    For each (b, h) and each chunk of at most ``chunk`` query rows, the scores
    against the keys visible to the chunk's last row are formed in one product.
    Scores of keys beyond a row's causal limit are then set to -inf, so their
    weight after the softmax is exactly 0.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, D) or v.shape != (B, S, Hkv, D):
        raise ValueError("k and v must be [B, S, Hkv, D] with q's B, S and D")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    s = default_scale(D) if scale is None else float(np.float32(scale))
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, dtype=np.int64)
    out = np.zeros((B, len(rows), len(heads), D), dtype=np.float64)
    for b in range(B):
        for hi, h in enumerate(heads):
            g = kv_head(int(h), Hq, Hkv)
            Kg = k[b, :, g, :]                       # [S, D]
            Vg = v[b, :, g, :]
            for c0 in range(0, len(rows), chunk):
                r = rows[c0:c0 + chunk]
                nvis = int(r.max()) + 1 if causal else S
                x = s * (q[b, r, h, :] @ Kg[:nvis].T)   # [len(r), nvis]
                if causal:
                    for ri, i in enumerate(r):
                        x[ri, i + 1:] = -np.inf
                p = _softmax_rows(x)
                out[b, c0:c0 + len(r), hi, :] = p @ Vg[:nvis]
    return out


def weights(q, k, causal: bool = True, scale: float | None = None) -> np.ndarray:
    """Attention weights P[b, h, i, j] for small inputs (zero where j is not visible to i)."""
    q = _as_f64(q)
    k = _as_f64(k)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    s = default_scale(D) if scale is None else float(np.float32(scale))
    P = np.zeros((B, Hq, S, S), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            for i in range(S):
                nvis = i + 1 if causal else S
                x = s * (k[b, :nvis, g, :] @ q[b, i, h, :])
                P[b, h, i, :nvis] = _softmax_rows(x[None, :])[0]
    return P


def decode(q, kcache, vcache, lens, scale: float | None = None) -> np.ndarray:
    """One query token per sequence against its KV cache.

    q: [B, Hq, D]; kcache, vcache: [B, L, Hkv, D]; lens: [B] ints.
    Sequence b sees cache slots 0..min(max(lens[b], 0), L)-1; slots beyond are
    never read, whatever they hold. An empty set gives a zero row.
    Returns float64 [B, Hq, D].
    """
    q = _as_f64(q)
    B, Hq, D = q.shape
    kc = np.asarray(kcache)
    vc = np.asarray(vcache)
    L, Hkv = kc.shape[1], kc.shape[2]
    if kc.shape != (B, L, Hkv, D) or vc.shape != (B, L, Hkv, D):
        raise ValueError("caches must be [B, L, Hkv, D]")
    s = default_scale(D) if scale is None else float(np.float32(scale))
    lens = np.asarray(lens, dtype=np.int64).reshape(B)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(min(max(lens[b], 0), L))
        if n == 0:
            continue
        Kb = _as_f64(kc[b, :n])                      # only the visible slots are widened
        Vb = _as_f64(vc[b, :n])
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            x = s * (Kb[:, g, :] @ q[b, h, :])       # [n]
            p = _softmax_rows(x[None, :])[0]
            out[b, h, :] = p @ Vb[:, g, :]
    return out


def decode_partials(q, kcache, vcache, lens, chunk: int, scale: float | None = None):
    """Split-KV decode, first half: attention of each chunk of the cache on its own.

    The cache axis is cut into nsplit = ceil(L / chunk) chunks of ``chunk``
    slots. Chunk c covers slots [c*chunk, min((c+1)*chunk, lens[b])).
    Returns (o_part [B, Hq, nsplit, D], lse [B, Hq, nsplit]), both float64:
    - o_part is the chunk's softmax-weighted average of V (normalized within
      the chunk);
    - lse is log(sum_j exp(x_j)) over the chunk, in natural-log units.
    An empty chunk has lse = -inf and o_part = 0.
    """
    q = _as_f64(q)
    B, Hq, D = q.shape
    kc = np.asarray(kcache)
    vc = np.asarray(vcache)
    L, Hkv = kc.shape[1], kc.shape[2]
    s = default_scale(D) if scale is None else float(np.float32(scale))
    nsplit = -(-L // chunk)
    lens = np.asarray(lens, dtype=np.int64).reshape(B)
    o_part = np.zeros((B, Hq, nsplit, D), dtype=np.float64)
    lse = np.full((B, Hq, nsplit), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(min(max(lens[b], 0), L))
        for c in range(nsplit):
            j0, j1 = c * chunk, min((c + 1) * chunk, n)
            if j1 <= j0:
                continue
            Kc = _as_f64(kc[b, j0:j1])
            Vc = _as_f64(vc[b, j0:j1])
            for h in range(Hq):
                g = kv_head(h, Hq, Hkv)
                x = s * (Kc[:, g, :] @ q[b, h, :])
                m = np.max(x)
                e = np.exp(x - m)
                tot = np.sum(e)
                o_part[b, h, c, :] = (e @ Vc[:, g, :]) / tot
                lse[b, h, c] = m + np.log(tot)
    return o_part, lse


def combine_partials(o_part, lse) -> np.ndarray:
    """Split-KV decode, second half: log-sum-exp merge of the chunks.

    out = sum_c w_c * o_c / sum_c w_c with w_c = exp(lse_c - M), where M is
    the largest finite lse. Chunks with lse = -inf get weight 0. If every
    chunk of a row is empty, the row is zero.
    o_part: [..., nsplit, D]; lse: [..., nsplit]. Returns [..., D].
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    finite = np.isfinite(lse)
    M = np.max(np.where(finite, lse, -np.inf), axis=-1, keepdims=True)
    anyf = np.any(finite, axis=-1, keepdims=True)
    Msafe = np.where(anyf, M, 0.0)
    w = np.where(finite, np.exp(np.where(finite, lse, 0.0) - Msafe), 0.0)
    num = np.sum(w[..., None] * o_part, axis=-2)
    den = np.sum(w, axis=-1)[..., None]
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
    return out
