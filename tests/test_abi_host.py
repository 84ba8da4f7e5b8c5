"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library must load, export every function include/gqa_attn.h declares, and
reject bad arguments with the documented codes before it makes any HIP call.
All pointers passed here are fake (never dereferenced): each call fails
validation before anything would touch them.
"""

import ctypes
import os
import re

import pytest

from gqa_flash_attention_amd import _lib
import gqa_flash_attention_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")

P = 0x10000      # a fake, 16-byte aligned "device pointer"
MIS = 0x10008    # a fake pointer that is not 16-byte aligned


@pytest.fixture(scope="module")
def lib():
    return _lib.get()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_attn_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strerror(lib):
    assert lib.gqa_attn_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -99):
        s = lib.gqa_attn_strerror(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.gqa_attn_last_error() == b""


def _prefill(lib, q=P, k=P, v=P, o=P, B=1, S=16, Hq=32, Hkv=8, D=128, scale=0.088, causal=1):
    return lib.gqa_attn_prefill(q, k, v, o, B, S, Hq, Hkv, D, scale, causal, None)


def test_prefill_argument_errors(lib):
    assert _prefill(lib, q=None) == _lib.ERR_NULL
    assert _prefill(lib, o=None) == _lib.ERR_NULL
    assert _prefill(lib, B=0) == _lib.ERR_DIM
    assert _prefill(lib, S=0) == _lib.ERR_DIM
    assert _prefill(lib, S=-5) == _lib.ERR_DIM
    assert _prefill(lib, Hq=0) == _lib.ERR_DIM
    assert _prefill(lib, Hkv=0) == _lib.ERR_DIM
    assert _prefill(lib, Hq=30, Hkv=8) == _lib.ERR_DIM
    assert _prefill(lib, scale=float("nan")) == _lib.ERR_DIM
    assert _prefill(lib, scale=float("inf")) == _lib.ERR_DIM
    assert _prefill(lib, D=64) == _lib.ERR_UNSUPPORTED
    assert _prefill(lib, D=256) == _lib.ERR_UNSUPPORTED
    assert _prefill(lib, q=MIS) == _lib.ERR_UNSUPPORTED
    assert _prefill(lib, v=MIS) == _lib.ERR_UNSUPPORTED
    assert _prefill(lib, o=MIS) == _lib.ERR_UNSUPPORTED
    # element counts past 2^62 are refused rather than wrapped
    assert _prefill(lib, B=2 ** 30, S=2 ** 30) == _lib.ERR_DIM


def test_prefill_tile_offset_bound(lib):
    # A full K/V tile is copied with 32-bit per-lane byte offsets r * Hkv * 256 + 16 * slot
    # (r < 64, slot < 16). The largest offset is 63 * Hkv * 256 + 255: below 2^32 up to
    # Hkv = 266305, so that head count is accepted and the next one refused (ERR_DIM, before
    # any HIP call; the pointers are fake and never touched).
    assert 63 * 266305 * 256 + 255 < 2 ** 32 <= 63 * 266306 * 256 + 255
    for Hkv, want in ((266305, 0), (266306, _lib.ERR_DIM), (1 << 20, _lib.ERR_DIM), ((1 << 31) - 1, _lib.ERR_DIM)):
        assert lib.gqa_attn_prefill_plan(1, 64, Hkv, Hkv, 128, None, None, None) == want, Hkv
        if want:
            assert _prefill(lib, S=64, Hq=Hkv, Hkv=Hkv) == want, Hkv
            assert lib.gqa_attn_prefill_form(P, P, P, P, 1, 64, Hkv, Hkv, 128, 0.088, 1, 4, 1, None) == want
    # row blocks x group size must stay below 2^31 - 16 (32-bit unit indices in the kernels)
    assert lib.gqa_attn_prefill_plan(1, 1 << 26, 1 << 10, 1, 128, None, None, None) == _lib.ERR_DIM
    assert lib.gqa_attn_prefill_plan(1, 1 << 20, 1 << 10, 1, 128, None, None, None) == 0


def test_prefill_form_argument_errors(lib):
    def form(waves, ks, q=P, B=1, S=16, D=128):
        return lib.gqa_attn_prefill_form(q, P, P, P, B, S, 32, 8, D, 0.088, 1, waves, ks, None)
    # only the three forms prefill_plan reports, or (0, 0) for the library's choice
    for waves, ks in ((4, 2), (8, 3), (12, 1), (16, 1), (2, 1), (0, 1), (4, 0), (-4, 1), (1, 1), (8, 0)):
        assert form(waves, ks) == _lib.ERR_UNSUPPORTED, (waves, ks)
    assert form(4, 1, q=None) == _lib.ERR_NULL
    assert form(8, 2, B=0) == _lib.ERR_DIM
    assert form(8, 1, D=64) == _lib.ERR_UNSUPPORTED
    assert form(4, 1, q=MIS) == _lib.ERR_UNSUPPORTED
    assert gqa.PREFILL_FORMS == ((4, 1), (8, 1), (8, 2))


def _decode(lib, q=P, k=P, v=P, lens=P, o=P, B=1, L=64, Hq=32, Hkv=8, D=128, scale=0.088):
    return lib.gqa_attn_decode(q, k, v, lens, o, B, L, Hq, Hkv, D, scale, None)


def test_decode_argument_errors(lib):
    assert _decode(lib, lens=None) == _lib.ERR_NULL
    assert _decode(lib, k=None) == _lib.ERR_NULL
    assert _decode(lib, B=0) == _lib.ERR_DIM
    assert _decode(lib, L=0) == _lib.ERR_DIM
    assert _decode(lib, Hq=12, Hkv=8) == _lib.ERR_DIM
    assert _decode(lib, scale=float("-inf")) == _lib.ERR_DIM
    assert _decode(lib, B=70000) == _lib.ERR_DIM          # grid z limit
    assert _decode(lib, D=96) == _lib.ERR_UNSUPPORTED
    assert _decode(lib, q=MIS) == _lib.ERR_UNSUPPORTED
    assert _decode(lib, k=MIS) == _lib.ERR_UNSUPPORTED


def test_decode_ws_and_split_errors(lib):
    need = lib.gqa_attn_decode_workspace_bytes(1, 1000, 32, 8, 128, 128)
    assert need > 0
    base = dict(q=P, k=P, v=P, lens=P, o=P)

    def call(chunk=128, ws=P, ws_bytes=need):
        return lib.gqa_attn_decode_ws(base["q"], base["k"], base["v"], base["lens"], base["o"],
                                      1, 1000, 32, 8, 128, 0.088, chunk, ws, ws_bytes, None)
    assert call(ws=None) == _lib.ERR_WORKSPACE
    assert call(ws=MIS) == _lib.ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == _lib.ERR_WORKSPACE
    for bad in (1, 63, 100, 96, -64):
        assert call(chunk=bad) == _lib.ERR_WORKSPACE, bad
    assert lib.gqa_attn_decode_workspace_bytes(1, 1000, 32, 8, 128, 100) == 0
    rc = lib.gqa_attn_decode_partials(P, P, P, P, 1, 1000, 32, 8, 128, 0.088, 128, P, need - 1, None)
    assert rc == _lib.ERR_WORKSPACE
    rc = lib.gqa_attn_decode_combine(P, 10, P, 1, 32, 128, 8, None)
    assert rc == _lib.ERR_WORKSPACE
    assert lib.gqa_attn_decode_combine(None, 10, P, 1, 32, 128, 8, None) == _lib.ERR_NULL
    assert lib.gqa_attn_decode_combine(P, 10 ** 9, P, 1, 32, 64, 8, None) == _lib.ERR_UNSUPPORTED
    assert lib.gqa_attn_decode_combine(P, 10 ** 9, P, 1, 32, 128, 0, None) == _lib.ERR_DIM
    # at most 2^18 splits per sequence, so one (sequence, KV head)'s partials fit 32-bit offsets
    big = (1 << 24) + 64   # 2^18 + 1 splits of 64 keys
    assert lib.gqa_attn_decode_workspace_bytes(1, big, 32, 8, 128, 64) == 0
    assert lib.gqa_attn_decode_workspace_bytes(1, big, 32, 8, 128, 128) > 0
    rc = lib.gqa_attn_decode_ws(P, P, P, P, P, 1, big, 32, 8, 128, 0.088, 64, P, 1 << 40, None)
    assert rc == _lib.ERR_WORKSPACE
    rc = lib.gqa_attn_decode_partials(P, P, P, P, 1, big, 32, 8, 128, 0.088, 64, P, 1 << 40, None)
    assert rc == _lib.ERR_WORKSPACE
    assert lib.gqa_attn_decode_combine(P, 1 << 40, P, 1, 32, 128, (1 << 18) + 1, None) == _lib.ERR_WORKSPACE
    # the fused decode's grid is splits x (KV heads x head groups) workgroups in one
    # dimension: 2^18 splits of 8192 KV heads (2^31 workgroups) is refused
    assert lib.gqa_attn_decode_workspace_bytes(1, 1 << 24, 8192, 8192, 128, 64) == 0
    assert lib.gqa_attn_decode_workspace_bytes(1, 1 << 24, 8192, 8192, 128, 128) > 0
    rc = lib.gqa_attn_decode_ws(P, P, P, P, P, 1, 1 << 24, 8192, 8192, 128, 0.088, 64, P, 1 << 40, None)
    assert rc == _lib.ERR_DIM


def test_decode_plan_and_workspace_size(lib):
    chunk = ctypes.c_int(0)
    nsplit = ctypes.c_int(0)
    for L in (1, 63, 64, 2048, 16384, 65536, 50001):
        assert lib.gqa_attn_decode_plan(1, L, 32, 8, 128, ctypes.byref(chunk), ctypes.byref(nsplit)) == 0
        assert chunk.value % 64 == 0 and 64 <= chunk.value <= 4096
        assert nsplit.value == -(-L // chunk.value)
        ws = lib.gqa_attn_decode_workspace_bytes(1, L, 32, 8, 128, 0)
        rows = 32 * nsplit.value
        counters = max(4096, 32)
        assert ws == ((counters * 4 + 255) // 256 * 256 + (rows * 128 * 4 + 255) // 256 * 256
                      + (rows * 4 + 255) // 256 * 256)
    # short caches: splits doubled up to 8 tiles while that leaves >= 128 workgroups
    for L, want in ((2048, 128), (3000, 128), (4096, 256), (6000, 192), (8192, 512), (12000, 384), (16384, 512)):
        assert lib.gqa_attn_decode_plan(1, L, 32, 8, 128, ctypes.byref(chunk), ctypes.byref(nsplit)) == 0
        assert chunk.value == want, (L, chunk.value)
    # batch-1 decodes of the workload are cut into about one chunk per CU (256 CUs)
    for L in (16384, 32768, 65536):
        assert lib.gqa_attn_decode_plan(1, L, 32, 8, 128, ctypes.byref(chunk), ctypes.byref(nsplit)) == 0
        assert nsplit.value * 8 == 256, (L, chunk.value, nsplit.value)
    # the library's own split stays within 2^18 splits up to L = 2^30
    assert lib.gqa_attn_decode_plan(1, 1 << 30, 32, 8, 128, ctypes.byref(chunk), ctypes.byref(nsplit)) == 0
    assert nsplit.value <= 1 << 18
    assert lib.gqa_attn_decode_plan(1, 100, 32, 8, 128, None, None) == 0
    assert lib.gqa_attn_decode_plan(0, 100, 32, 8, 128, None, None) == _lib.ERR_DIM


def test_prefill_plan(lib):
    waves = ctypes.c_int(0)
    wgs = ctypes.c_int(0)
    ks = ctypes.c_int(0)
    # batch 1, Llama-3-8B heads: (waves, key splits, units per workgroup). 4 units of one
    # wave each below 512 keys; the key split (4 units x 2 waves) up to 2048 keys, while
    # the 4-unit grid holds at most 2 workgroups per CU; 4 units again up to 3392 (the
    # 8-unit grid below 5/3 workgroups per CU); then 8.
    for S, want in ((1, (4, 1, 4)), (511, (4, 1, 4)), (512, (8, 2, 4)), (1000, (8, 2, 4)),
                    (2048, (8, 2, 4)), (2049, (4, 1, 4)), (3392, (4, 1, 4)), (3393, (8, 1, 8)),
                    (4096, (8, 1, 8)), (8128, (8, 1, 8)),
                    (8129, (8, 1, 8)), (8192, (8, 1, 8)), (32768, (8, 1, 8))):
        assert lib.gqa_attn_prefill_plan(1, S, 32, 8, 128, ctypes.byref(waves), ctypes.byref(wgs),
                                         ctypes.byref(ks)) == 0
        assert (waves.value, ks.value) == want[:2], S
        units = 4 * -(-S // 32)
        assert wgs.value == 8 * -(-units // want[2]), S
    # a batch reaches the thresholds sooner: at S = 1000, 8 units from B = 4 (512 8-unit
    # workgroups), 4 units at B = 3 (384 of them, and 768 4-unit ones: no key split)
    assert lib.gqa_attn_prefill_plan(8, 1000, 32, 8, 128, ctypes.byref(waves), None, ctypes.byref(ks)) == 0
    assert (waves.value, ks.value) == (8, 1)
    assert lib.gqa_attn_prefill_plan(4, 1000, 32, 8, 128, ctypes.byref(waves), None, ctypes.byref(ks)) == 0
    assert (waves.value, ks.value) == (8, 1)
    assert lib.gqa_attn_prefill_plan(3, 1000, 32, 8, 128, ctypes.byref(waves), None, ctypes.byref(ks)) == 0
    assert (waves.value, ks.value) == (4, 1)
    assert lib.gqa_attn_prefill_plan(2, 1000, 32, 8, 128, ctypes.byref(waves), None, ctypes.byref(ks)) == 0
    assert (waves.value, ks.value) == (8, 2)
    assert lib.gqa_attn_prefill_plan(1, 100, 32, 8, 128, None, None, None) == 0
    assert lib.gqa_attn_prefill_plan(0, 100, 32, 8, 128, None, None, None) == _lib.ERR_DIM
    assert lib.gqa_attn_prefill_plan(1, 100, 32, 8, 64, None, None, None) == _lib.ERR_UNSUPPORTED
    assert lib.gqa_attn_prefill_plan(1, 100, 30, 8, 128, None, None, None) == _lib.ERR_DIM


def test_release_without_any_workspace_is_harmless(lib):
    lib.gqa_attn_release()


def test_probe_argument_errors(lib):
    # HBM read probe: buf, bytes (multiple of 16), workgroups, sink (>= 256 words per workgroup)
    assert lib.gqa_attn_probe_hbm_read(None, 1024, 4, P, 1024, None) == _lib.ERR_NULL
    assert lib.gqa_attn_probe_hbm_read(P, 1024, 4, None, 1024, None) == _lib.ERR_NULL
    assert lib.gqa_attn_probe_hbm_read(P, 0, 4, P, 1024, None) == _lib.ERR_DIM
    assert lib.gqa_attn_probe_hbm_read(P, 1000, 4, P, 1024, None) == _lib.ERR_DIM
    assert lib.gqa_attn_probe_hbm_read(P, 1024, 0, P, 1024, None) == _lib.ERR_DIM
    assert lib.gqa_attn_probe_hbm_read(P, 1024, 65536, P, 1 << 30, None) == _lib.ERR_DIM
    assert lib.gqa_attn_probe_hbm_read(MIS, 1024, 4, P, 1024, None) == _lib.ERR_UNSUPPORTED
    assert lib.gqa_attn_probe_hbm_read(P, 1024, 4, P, 1023, None) == _lib.ERR_WORKSPACE
    # MFMA probe: rounds, seed, workgroups, sink (>= 256 per workgroup), ticks (>= 2 per workgroup)
    assert lib.gqa_attn_probe_mfma_bf16(8, 1, 512, None, 1 << 17, P, 1024, None) == _lib.ERR_NULL
    assert lib.gqa_attn_probe_mfma_bf16(8, 1, 512, P, 1 << 17, None, 1024, None) == _lib.ERR_NULL
    assert lib.gqa_attn_probe_mfma_bf16(0, 1, 512, P, 1 << 17, P, 1024, None) == _lib.ERR_DIM
    assert lib.gqa_attn_probe_mfma_bf16((1 << 20) + 1, 1, 512, P, 1 << 17, P, 1024, None) == _lib.ERR_DIM
    assert lib.gqa_attn_probe_mfma_bf16(8, 1, 0, P, 1 << 17, P, 1024, None) == _lib.ERR_DIM
    assert lib.gqa_attn_probe_mfma_bf16(8, 1, 512, P, (1 << 17) - 1, P, 1024, None) == _lib.ERR_WORKSPACE
    assert lib.gqa_attn_probe_mfma_bf16(8, 1, 512, P, 1 << 17, P, 1023, None) == _lib.ERR_WORKSPACE


def test_decode_noalloc_argument_errors(lib):
    def call(q=P, k=P, v=P, lens=P, o=P, B=1, L=64, Hq=32, Hkv=8, D=128, scale=0.088):
        return lib.gqa_attn_decode_noalloc(q, k, v, lens, o, B, L, Hq, Hkv, D, scale, None)
    assert call(lens=None) == _lib.ERR_NULL
    assert call(o=None) == _lib.ERR_NULL
    assert call(B=0) == _lib.ERR_DIM
    assert call(Hq=12) == _lib.ERR_DIM
    assert call(D=64) == _lib.ERR_UNSUPPORTED
    assert call(k=MIS) == _lib.ERR_UNSUPPORTED
    # the per-GPU scratch holds 8 MiB: a batch-1 decode of 2^21 keys needs 8.08 MiB and is
    # refused before any HIP call, with the sizes in the error detail
    assert lib.gqa_attn_decode_workspace_bytes(1, 1 << 21, 32, 8, 128, 0) > 8 << 20
    assert lib.gqa_attn_decode_workspace_bytes(1, 1 << 20, 32, 8, 128, 0) <= 8 << 20
    assert call(L=1 << 21) == _lib.ERR_WORKSPACE
    assert b"scratch" in lib.gqa_attn_last_error()
    assert call(B=64, L=50000) == _lib.ERR_WORKSPACE


def test_prefill_tiles_argument_errors(lib):
    def tiles(bm, bn, nw, q=P, B=1, S=16, Hq=32, Hkv=8, D=128):
        return lib.gqa_attn_prefill_tiles(q, P, P, P, B, S, Hq, Hkv, D, 0.088, 1, bm, bn, nw, None)
    for bm, bn, nw in ((32, 16, 4), (32, 256, 4), (64, 128, 4), (64, 64, 8), (16, 64, 4), (32, 64, 2),
                       (32, 32, 16), (0, 0, 0), (96, 64, 4)):
        assert tiles(bm, bn, nw) == _lib.ERR_UNSUPPORTED, (bm, bn, nw)
    assert tiles(32, 32, 4, q=None) == _lib.ERR_NULL
    assert tiles(64, 64, 4, B=0) == _lib.ERR_DIM
    assert tiles(32, 128, 8, D=64) == _lib.ERR_UNSUPPORTED
    assert tiles(32, 32, 8, q=MIS) == _lib.ERR_UNSUPPORTED
    # 128-key tiles address rows up to 127 with 32-bit offsets: Hkv <= 132104
    assert 127 * 132104 * 256 + 255 < 2 ** 32 <= 127 * 132105 * 256 + 255
    assert tiles(32, 128, 4, S=64, Hq=132105, Hkv=132105) == _lib.ERR_DIM
    assert tiles(32, 128, 4, S=64, Hq=132105, Hkv=132105, q=MIS) == _lib.ERR_DIM
