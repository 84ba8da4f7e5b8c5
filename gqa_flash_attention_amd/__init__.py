"""GQA attention forward for MI355X (gfx950): thin Python binding over libgqa_attn.so.

Every step of the computation runs in the HIP kernels behind the C ABI
(include/gqa_attn.h). This module only checks tensors, allocates outputs with
torch, and passes raw device pointers plus torch's current HIP stream.

    out = prefill(q, k, v, causal=True)   # q [B,S,Hq,128], k/v [B,S,Hkv,128] bf16
    out = decode(q, kcache, vcache, lens) # q [B,Hq,128], caches [B,L,Hkv,128], lens int32 [B]
"""

from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import GqaAttnError  # noqa: F401

__all__ = [
    "prefill", "prefill_plan", "decode", "decode_noalloc", "decode_plan", "decode_workspace_bytes", "decode_workspace",
    "decode_partials", "decode_combine", "default_scale", "release", "version", "GqaAttnError",
]

D_SUPPORTED = 128


def default_scale(D: int) -> float:
    """1/sqrt(D) rounded to float32: the scale used when none is given."""
    return ctypes.c_float(1.0 / math.sqrt(D)).value


def _stream_ptr(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_workspace(ws, device) -> None:
    """A caller-owned workspace: a contiguous uint8 tensor on the device of the call (the
    library checks its size and 16-byte alignment)."""
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if not ws.is_cuda or ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")


def _check_bf16(name: str, t: torch.Tensor, ndim: int, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
            scale: float | None = None, out: torch.Tensor | None = None,
            form: tuple[int, int] | None = None, tiles: tuple[int, int, int] | None = None) -> torch.Tensor:
    """Attention over a prompt. q [B,S,Hq,D], k/v [B,S,Hkv,D] -> out [B,S,Hq,D] (bf16).

    ``form`` = (waves, key_splits), one of the pairs prefill_plan reports ((4, 1), (8, 1)
    or (8, 2)), runs that workgroup form whatever the shape; ``tiles`` =
    (rows_per_wave, keys_per_tile, waves), one of PREFILL_TILES, runs that tile shape;
    with neither the library chooses.
    """
    _check_bf16("q", q, 4)
    _check_bf16("k", k, 4, q.device)
    _check_bf16("v", v, 4, q.device)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, D) or tuple(v.shape) != (B, S, Hkv, D):
        raise ValueError(f"k/v must be [B, S, Hkv, D] = [{B}, {S}, Hkv, {D}], got {tuple(k.shape)} and {tuple(v.shape)}")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16("out", out, 4, q.device)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if scale is None:
        scale = default_scale(D)
    if form is not None and tiles is not None:
        raise ValueError("give form or tiles, not both")
    with torch.cuda.device(q.device):
        if tiles is not None:
            bm, bn, nw = (int(x) for x in tiles)
            rc = _lib.get().gqa_attn_prefill_tiles(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                   B, S, Hq, Hkv, D, float(scale), 1 if causal else 0,
                                                   bm, bn, nw, _stream_ptr(q))
            _lib.check(rc, "gqa_attn_prefill_tiles")
            return out
        if form is None:
            rc = _lib.get().gqa_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                             B, S, Hq, Hkv, D, float(scale), 1 if causal else 0, _stream_ptr(q))
        else:
            waves, ks = (int(x) for x in form)
            rc = _lib.get().gqa_attn_prefill_form(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                  B, S, Hq, Hkv, D, float(scale), 1 if causal else 0,
                                                  waves, ks, _stream_ptr(q))
    _lib.check(rc, "gqa_attn_prefill_form" if form is not None else "gqa_attn_prefill")
    return out


def _check_decode(q, kcache, vcache, lens):
    _check_bf16("q", q, 3)
    _check_bf16("kcache", kcache, 4, q.device)
    _check_bf16("vcache", vcache, 4, q.device)
    B, Hq, D = q.shape
    L, Hkv = kcache.shape[1], kcache.shape[2]
    if tuple(kcache.shape) != (B, L, Hkv, D) or tuple(vcache.shape) != (B, L, Hkv, D):
        raise ValueError(f"caches must be [B, L, Hkv, D] with B={B}, D={D}")
    if not isinstance(lens, torch.Tensor) or lens.dtype != torch.int32 or lens.dim() != 1 \
            or lens.shape[0] != B or lens.device != q.device or not lens.is_contiguous():
        raise ValueError("lens must be a contiguous int32 tensor [B] on q's device")
    return B, L, Hq, Hkv, D


def decode(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor, lens: torch.Tensor,
           scale: float | None = None, out: torch.Tensor | None = None,
           chunk: int | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One-token decode. q [B,Hq,D], caches [B,L,Hkv,D], lens int32 [B] -> out [B,Hq,D] (bf16).

    With neither ``chunk`` nor ``workspace`` the library picks the split and uses
    its own cached workspace; otherwise a torch-owned workspace is used (allocated
    and zeroed here if not given) with the requested keys per split. A workspace
    passed in must have been allocated zeroed (decode_workspace() returns one): its
    leading merge counters must be zero, and every completed call leaves them zero.
    """
    B, L, Hq, Hkv, D = _check_decode(q, kcache, vcache, lens)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16("out", out, 3, q.device)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if scale is None:
        scale = default_scale(D)
    lib = _lib.get()
    if workspace is not None:
        _check_workspace(workspace, q.device)
    with torch.cuda.device(q.device):
        if chunk is None and workspace is None:
            rc = lib.gqa_attn_decode(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), lens.data_ptr(),
                                     out.data_ptr(), B, L, Hq, Hkv, D, float(scale), _stream_ptr(q))
            _lib.check(rc, "gqa_attn_decode")
            return out
        ch = 0 if chunk is None else int(chunk)
        if workspace is None:
            workspace = decode_workspace(B, L, Hq, Hkv, D, ch, device=q.device)
        rc = lib.gqa_attn_decode_ws(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), lens.data_ptr(),
                                    out.data_ptr(), B, L, Hq, Hkv, D, float(scale), ch,
                                    workspace.data_ptr(), workspace.numel(), _stream_ptr(q))
    _lib.check(rc, "gqa_attn_decode_ws")
    return out


def decode_noalloc(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor, lens: torch.Tensor,
                   out: torch.Tensor, scale: float | None = None) -> torch.Tensor:
    """decode() through gqa_attn_decode_noalloc: the library allocates nothing (its split
    partials live in a fixed 8 MiB scratch per GPU, shared by every call on that GPU, so
    overlapping calls on one GPU race). The caller passes `out` [B,Hq,D] bf16."""
    B, L, Hq, Hkv, D = _check_decode(q, kcache, vcache, lens)
    _check_bf16("out", out, 3, q.device)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if scale is None:
        scale = default_scale(D)
    with torch.cuda.device(q.device):
        rc = _lib.get().gqa_attn_decode_noalloc(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), lens.data_ptr(),
                                                out.data_ptr(), B, L, Hq, Hkv, D, float(scale), _stream_ptr(q))
    _lib.check(rc, "gqa_attn_decode_noalloc")
    return out


# The workgroup forms of the prefill as (waves, key_splits): 4 units of one wave, 8 units of one
# wave, 4 units of two waves that split the key tiles.
PREFILL_FORMS = ((4, 1), (8, 1), (8, 2))
# The tile shapes gqa_attn_prefill_tiles runs, as (rows per wave, keys per tile, waves per
# workgroup); the first two are the library's own 4- and 8-wave forms.
PREFILL_TILES = ((32, 64, 4), (32, 64, 8), (32, 32, 4), (32, 32, 8), (32, 128, 4), (32, 128, 8),
                 (64, 32, 4), (64, 64, 4))


def prefill_plan(B: int, S: int, Hq: int, Hkv: int, D: int = D_SUPPORTED):
    """(waves per workgroup, workgroups, key splits) the library launches for this prefill shape."""
    waves = ctypes.c_int(0)
    wgs = ctypes.c_int(0)
    ks = ctypes.c_int(0)
    rc = _lib.get().gqa_attn_prefill_plan(B, S, Hq, Hkv, D, ctypes.byref(waves), ctypes.byref(wgs),
                                          ctypes.byref(ks))
    _lib.check(rc, "gqa_attn_prefill_plan")
    return waves.value, wgs.value, ks.value


def decode_plan(B: int, L: int, Hq: int, Hkv: int, D: int = D_SUPPORTED):
    """(keys per split, number of splits) the library chooses for this shape."""
    chunk = ctypes.c_int(0)
    nsplit = ctypes.c_int(0)
    rc = _lib.get().gqa_attn_decode_plan(B, L, Hq, Hkv, D, ctypes.byref(chunk), ctypes.byref(nsplit))
    _lib.check(rc, "gqa_attn_decode_plan")
    return chunk.value, nsplit.value


def decode_workspace_bytes(B: int, L: int, Hq: int, Hkv: int, D: int = D_SUPPORTED, chunk: int = 0) -> int:
    return int(_lib.get().gqa_attn_decode_workspace_bytes(B, L, Hq, Hkv, D, chunk))


def decode_workspace(B: int, L: int, Hq: int, Hkv: int, D: int = D_SUPPORTED, chunk: int = 0,
                     device=None) -> torch.Tensor:
    """A zeroed workspace for decodes of this shape with `chunk` keys per split (0 = the
    library's choice), allocated by torch on `device` (default: the current GPU)."""
    need = int(_lib.get().gqa_attn_decode_workspace_bytes(B, L, Hq, Hkv, D, int(chunk)))
    if need == 0:
        raise GqaAttnError(_lib.ERR_WORKSPACE, "gqa_attn_decode_workspace_bytes")
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    return torch.zeros(need, dtype=torch.uint8, device=dev)


def _split_views(ws: torch.Tensor, B: int, Hq: int, nsplit: int, D: int):
    # workspace layout (include/gqa_attn.h): counters | o_part | lse, 256-byte aligned parts
    rows = B * Hq * nsplit
    o_off = (max(4096, B * Hq) * 4 + 255) // 256 * 256
    lse_off = o_off + (rows * D * 4 + 255) // 256 * 256
    o_part = ws[o_off: o_off + rows * D * 4].view(torch.float32).view(B, Hq, nsplit, D)
    lse = ws[lse_off: lse_off + rows * 4].view(torch.float32).view(B, Hq, nsplit)
    return o_part, lse


def decode_partials(q, kcache, vcache, lens, chunk: int, scale: float | None = None):
    """The split half of a decode: (o_part [B,Hq,nsplit,D] fp32, lse [B,Hq,nsplit] fp32, log2 units,
    workspace). Chunks with lse = -inf are empty and their o_part rows are unspecified."""
    B, L, Hq, Hkv, D = _check_decode(q, kcache, vcache, lens)
    if scale is None:
        scale = default_scale(D)
    lib = _lib.get()
    need = int(lib.gqa_attn_decode_workspace_bytes(B, L, Hq, Hkv, D, int(chunk)))
    if need == 0:
        raise GqaAttnError(_lib.ERR_WORKSPACE, "gqa_attn_decode_workspace_bytes")
    ws = torch.zeros(need, dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        rc = lib.gqa_attn_decode_partials(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), lens.data_ptr(),
                                          B, L, Hq, Hkv, D, float(scale), int(chunk), ws.data_ptr(), need,
                                          _stream_ptr(q))
    _lib.check(rc, "gqa_attn_decode_partials")
    nsplit = -(-L // int(chunk))
    o_part, lse = _split_views(ws, B, Hq, nsplit, D)
    return o_part, lse, ws


def decode_combine(ws: torch.Tensor, B: int, Hq: int, nsplit: int, D: int = D_SUPPORTED,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """The merge half of a decode: workspace (as written by decode_partials) -> out [B,Hq,D] bf16."""
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda:
        raise ValueError("ws must be a GPU tensor (the workspace decode_partials returned)")
    _check_workspace(ws, ws.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=ws.device)
    else:
        _check_bf16("out", out, 3, ws.device)
        if tuple(out.shape) != (B, Hq, D):
            raise ValueError(f"out must be [{B}, {Hq}, {D}]")
    with torch.cuda.device(ws.device):
        rc = _lib.get().gqa_attn_decode_combine(ws.data_ptr(), ws.numel(), out.data_ptr(),
                                                B, Hq, D, nsplit, _stream_ptr(out))
    _lib.check(rc, "gqa_attn_decode_combine")
    return out


def release() -> None:
    """Free the library's cached decode workspaces (synchronise first)."""
    _lib.get().gqa_attn_release()


def version() -> int:
    return int(_lib.get().gqa_attn_version())
