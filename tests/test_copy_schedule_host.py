"""A host-side model of the HBM -> LDS copy schedules of the three prefill forms and the
two decode kernels, checked over a set of shapes (no GPU involved).

The model restates, step by step, what the kernels' loops do with their copies: which K/V
tile each wave copies at which step, into which LDS ring stage, from which global rows,
and where each wave waits and meets a barrier (prefill.hip: prefill_kernel,
prefill_split_kernel, prefill_tiles_kernel with TileCopyN and stage_tile_n; decode.hip:
decode_kernel; gqa_device.hpp: TileCopy and stage_tile). It checks, for every copy instruction and every lane:
- the global bytes read lie inside the K or V tensor (row < S, or < lens[b] for a
  decode), and a full-tile copy's 32-bit byte offset does not wrap;
- a full tile's 16 chunks x 64 rows are each fetched exactly once, into the LDS slot the
  read side (lds_read_k / lds_read_v_tr swizzles) looks them up at;
- no copy is issued into a ring stage that a wave may still read for an older tile,
  and no two copies in flight at once target the same stage;
- every tile a wave reads was waited for (its copies complete and published by a
  barrier) before the read;
- the decode's splits cover every key of every sequence exactly once.
"""

import itertools

import pytest

TILE = 64
ROW_BYTES = 256


def swz_k(r):
    return r & 15


def swz_v(r):
    return (6 if r & 1 else 0) ^ (10 if r & 2 else 0)


def tilecopy_offsets(NW, wave, row_stride_elems):
    """TileCopy<NW>::init: per instruction j, per lane: (row r, chunk c, byte offset, LDS byte)."""
    out = []
    for j in range((TILE // 4) // NW):
        for lane in range(64):
            r = 4 * (wave + NW * j) + (lane >> 4)
            slot = lane & 15
            row = r * row_stride_elems * 2
            out.append(("K", r, slot ^ swz_k(r), row + ((slot ^ swz_k(r)) << 4), (wave + NW * j) * 1024 + 16 * lane))
            out.append(("V", r, slot ^ swz_v(r), row + ((slot ^ swz_v(r)) << 4), (wave + NW * j) * 1024 + 16 * lane))
    return out


@pytest.mark.parametrize("NW", [4, 8])
def test_full_tile_copy_is_a_bijection_onto_the_swizzled_layout(NW):
    Hkv = 8
    seen = {"K": set(), "V": set()}
    for wave in range(NW):
        for kind, r, c, off, lds in tilecopy_offsets(NW, wave, Hkv * 128):
            assert 0 <= r < TILE and 0 <= c < 16
            assert off == r * Hkv * ROW_BYTES + 16 * c          # global: row r, chunk c of this head
            swz = swz_k(r) if kind == "K" else swz_v(r)
            assert lds == r * ROW_BYTES + ((c ^ swz) << 4)       # where lds_read_k / lds_read_v_tr look
            assert (r, c) not in seen[kind]
            seen[kind].add((r, c))
    assert len(seen["K"]) == len(seen["V"]) == TILE * 16


@pytest.mark.parametrize("NW", [4, 8])
def test_every_wave_issues_the_same_number_of_copies_per_tile_full_or_ragged(NW):
    # the decode waits with vmcnt = (tiles still allowed in flight) x (copies per wave per
    # tile), so a ragged tile must cost each wave as many copy instructions as a full one
    full = 2 * ((TILE // 4) // NW)                              # TileCopy<NW>: K and V
    for wave in range(NW):
        ragged = 2 * len(range(wave, TILE // 4, NW))            # stage_tile<NW>: K and V
        assert ragged == full


@pytest.mark.parametrize("Hkv", [1, 8, 1000, 266305])
def test_full_tile_offsets_fit_32_bits_for_every_accepted_head_count(Hkv):
    # the library accepts Hkv <= 266305 (plan_prefill); the largest offset then fits
    worst = max(off for wave in range(4) for _, _, _, off, _ in tilecopy_offsets(4, wave, Hkv * 128))
    assert worst == 63 * Hkv * ROW_BYTES + 15 * 16     # row 63, chunk 15: its 16 bytes end below 2^32
    assert worst + 16 <= 2 ** 32


def stage_tile_rows(nvalid, NW, wave):
    """stage_tile: the global row each lane of each instruction of `wave` reads."""
    rows = []
    for i in range(wave, TILE // 4, NW):
        for lane in range(64):
            r = 4 * i + (lane >> 4)
            rows.append(r if r < nvalid else nvalid - 1)
    return rows


class Ring:
    """LDS ring stages: which tile each holds, which copies are in flight, who reads."""

    def __init__(self, nstage):
        self.tile = [None] * nstage        # tile whose data the stage holds or is receiving
        self.inflight = [False] * nstage   # a copy into the stage not yet waited for
        self.published = [False] * nstage  # copy complete and a barrier passed since
        self.readers = [set() for _ in range(nstage)]   # waves that may still read it

    def issue(self, st, tile):
        assert not self.inflight[st], f"two copies in flight into stage {st}"
        assert not self.readers[st], f"stage {st} refilled while waves {self.readers[st]} may still read tile {self.tile[st]}"
        self.tile[st], self.inflight[st], self.published[st] = tile, True, False

    def wait_all(self):
        for s in range(len(self.tile)):
            if self.inflight[s]:
                self.inflight[s] = False
                self.published[s] = "pending"

    def barrier(self):
        for s in range(len(self.tile)):
            if self.published[s] == "pending":
                self.published[s] = True
            self.readers[s].clear()   # every wave has finished the reads it issued before

    def read(self, st, tile, wave):
        assert self.tile[st] == tile, f"stage {st} holds tile {self.tile[st]}, wave {wave} reads {tile}"
        assert self.published[st] is True, f"tile {tile} read before its copy was waited for and published"
        self.readers[st].add(wave)


def stage_tile_rows_n(nvalid, NW, wave, bn):
    """stage_tile_n<NW, BN>: the global row each lane of each instruction of `wave` reads."""
    rows = []
    for i in range(wave, bn // 4, NW):
        for lane in range(64):
            r = 4 * i + (lane >> 4)
            rows.append(r if r < nvalid else nvalid - 1)
    return rows


def check_rows_in_bounds(t, kv_end, S, NW, bn=TILE):
    r0 = t * bn
    assert 0 <= t and r0 < kv_end <= S
    if kv_end - r0 >= bn:
        assert r0 + bn <= S                        # full tile: rows r0 .. r0+bn-1
    else:
        for w in range(NW):
            for r in stage_tile_rows_n(kv_end - r0, NW, w, bn):
                assert 0 <= r0 + r < kv_end        # ragged tile: clamped to the last valid row


def prefill_workgroup(NW, S, G, wg, causal=True, bn=TILE, nq=1):
    """prefill_kernel<causal, *, NW> (bn = 64, nq = 1) or prefill_tiles_kernel<causal, *, NW,
    bn / 32, nq>: the tiles one workgroup copies and reads, in order."""
    P = max(1, 64 * (NW // 4) * nq // bn)
    NST = 2 * P
    nrb = -(-S // 32)
    nunits = G * nrb
    per_wg = NW * nq
    last_unit = min(per_wg * wg + per_wg - 1, nunits - 1)
    kv_end = min(S, (last_unit // G) * 32 + 32) if causal else S
    nt = -(-kv_end // bn)
    ring = Ring(NST)
    own_nt = {}
    for w in range(NW):
        own_nt[w] = 0
        for u in range(nq):
            unit = nq * (NW * wg + w) + u
            if unit < nunits:
                q0 = (unit // G) * 32
                own_nt[w] = max(own_nt[w], -(-(min(S, q0 + 32) if causal else S) // bn))
    assert max(own_nt.values()) <= nt

    def issue(t, st):
        check_rows_in_bounds(t, kv_end, S, NW, bn)
        ring.issue(st, t)

    issue(0, 0)
    ring.wait_all()
    for t in range(1, P):
        if t < nt:
            issue(t, t)
    for t in range(nt):
        BUF = t % NST
        if BUF % P == 0:
            ring.wait_all()
            ring.barrier()
            for i in range(P):
                if t + P + i < nt:
                    issue(t + P + i, (BUF + P + i) % NST)
        for w in range(NW):
            if t < own_nt[w]:
                ring.read(BUF, t, w)
    return nt


def prefill_split_workgroup(S, G, wg, causal=True):
    """prefill_split_kernel: two halves of 4 waves, each with a 2-stage ring of its own."""
    nrb = -(-S // 32)
    nunits = G * nrb
    last_unit = min(4 * wg + 3, nunits - 1)
    kv_end = min(S, (last_unit // G) * 32 + 32) if causal else S
    nt = -(-kv_end // TILE)
    mid = (nt + 1) // 2
    rings = [Ring(2), Ring(2)]
    bounds = [(0, mid), (mid, nt)]
    for h in (0, 1):
        tb, te = bounds[h]
        if tb < te:
            check_rows_in_bounds(tb, kv_end, S, 4)
            rings[h].issue(0, tb)
        rings[h].wait_all()
    for i in range(mid):
        for h in (0, 1):
            rings[h].wait_all()
        for h in (0, 1):
            rings[h].barrier()
        for h in (0, 1):
            tb, te = bounds[h]
            t = tb + i
            if t + 1 < te:
                check_rows_in_bounds(t + 1, kv_end, S, 4)
                rings[h].issue((i % 2) ^ 1, t + 1)
            if t < te:
                for w in range(4):
                    rings[h].read(i % 2, t, (h, w))
    return nt


PREFILL_SHAPES = [(1, 8), (63, 4), (64, 4), (65, 4), (127, 4), (300, 4), (1000, 4), (3000, 4), (4096, 4), (5000, 1),
                  (700, 32), (161, 16)]


@pytest.mark.parametrize("NW", [4, 8])
@pytest.mark.parametrize("S,G", PREFILL_SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_copy_schedule(NW, S, G, causal):
    units = G * -(-S // 32)
    for wg in range(-(-units // NW)):
        prefill_workgroup(NW, S, G, wg, causal)


@pytest.mark.parametrize("bm,bn,NW", [(32, 32, 4), (32, 32, 8), (32, 128, 4), (32, 128, 8), (64, 32, 4),
                                      (64, 64, 4)])
@pytest.mark.parametrize("S,G", PREFILL_SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_tile_shape_copy_schedule(bm, bn, NW, S, G, causal):
    nq = bm // 32
    units = G * -(-S // 32)
    for wg in range(-(-units // (NW * nq))):
        prefill_workgroup(NW, S, G, wg, causal, bn=bn, nq=nq)


@pytest.mark.parametrize("NW,bn", [(4, 32), (8, 32), (4, 128), (8, 128)])
def test_tile_copy_n_is_a_bijection(NW, bn):
    seen = {"K": set(), "V": set()}
    for wave in range(NW):
        for j in range((bn // 4) // NW):
            for lane in range(64):
                r = 4 * (wave + NW * j) + (lane >> 4)
                slot = lane & 15
                for kind, swz in (("K", swz_k(r)), ("V", swz_v(r))):
                    c = slot ^ swz
                    assert (wave + NW * j) * 1024 + 16 * lane == r * ROW_BYTES + ((c ^ swz) << 4)
                    assert (r, c) not in seen[kind]
                    seen[kind].add((r, c))
    assert len(seen["K"]) == len(seen["V"]) == bn * 16


@pytest.mark.parametrize("S,G", PREFILL_SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_split_copy_schedule(S, G, causal):
    units = G * -(-S // 32)
    for wg in range(-(-units // 4)):
        prefill_split_workgroup(S, G, wg, causal)


DEC_WAVES = 4        # decode waves that attend (16 keys of each tile each)
DEC_COPY_WAVES = 8   # decode waves that issue the tile copies


def decode_workgroup(L, length, nsplit, chunk, split, strided, nstage=4):
    """decode_kernel<nstage, fused, strided> for one split: the keys of each tile it streams.
    All DEC_COPY_WAVES waves issue copies and meet every tile barrier; the first DEC_WAVES
    read the tiles."""
    T = -(-length // TILE)
    if strided:
        ntiles = (T - 1 - split) // nsplit + 1 if split < T else 0
        key = lambda t: (t * nsplit + split) * TILE
    else:
        nkeys = min(chunk, length - split * chunk)
        ntiles = -(-nkeys // TILE) if nkeys > 0 else 0
        rot = (5 * split) % ntiles if ntiles > 0 else 0
        key = lambda t: split * chunk + ((t + rot) if t + rot < ntiles else t + rot - ntiles) * TILE
    ring = Ring(nstage)
    keys = []

    def issue(t):
        r0 = key(t)
        assert 0 <= r0 < length <= L
        if length - r0 >= TILE:
            assert r0 + TILE <= length
        else:
            for w in range(DEC_COPY_WAVES):
                for r in stage_tile_rows(length - r0, DEC_COPY_WAVES, w):
                    assert 0 <= r0 + r < length
        ring.issue(t % nstage, t)

    for t in range(min(nstage - 1, ntiles)):
        issue(t)
    issued = min(nstage - 1, ntiles)           # tiles issued so far (0 .. issued-1)
    for t in range(ntiles):
        # wait_tiles_ahead(ahead): each wave's copies complete in issue order, so all but
        # the copies of its `ahead` most recently issued tiles have landed
        ahead = min(nstage - 2, ntiles - 1 - t)
        for s in range(nstage):
            if ring.inflight[s] and ring.tile[s] < issued - ahead:
                ring.inflight[s] = False
                ring.published[s] = "pending"
        ring.barrier()
        if t + nstage - 1 < ntiles:
            issue(t + nstage - 1)
            issued += 1
        ks = key(t)
        for w in range(DEC_WAVES):
            if ks + 16 * w < length:
                ring.read(t % nstage, t, w)
        keys.extend(range(ks, min(ks + TILE, length)))
    return keys


@pytest.mark.parametrize("L,lens,chunk", [(64, [64, 1], 64), (65, [65], 64), (1000, [1000, 357, 0], 128),
                                          (5000, [5000, 4999, 1], 256), (16384, [16384], 512),
                                          (50001, [50001, 12345, 64, 63], 4096), (777, [777], 832),
                                          (3000, [3000], 3008), (20000, [20000, 7001], 4096)])
@pytest.mark.parametrize("strided", [True, False])
def test_decode_copy_schedule_and_key_coverage(L, lens, chunk, strided):
    nsplit = -(-L // chunk)
    for length in lens:
        covered = []
        for split in range(nsplit):
            covered += decode_workgroup(L, length, nsplit, chunk, split, strided)
        assert sorted(covered) == list(range(length)), "every key of the sequence exactly once"


def test_the_model_rejects_the_mistakes_it_looks_for():
    # a copy of a tile past the last one (the bound dropped from an issue guard)
    with pytest.raises(AssertionError):
        check_rows_in_bounds(5, kv_end=300, S=300, NW=4)
    # a second copy into a stage whose first copy has not been waited for
    r = Ring(2)
    r.issue(0, 0)
    with pytest.raises(AssertionError):
        r.issue(0, 2)
    # refilling a stage another wave may still read
    r = Ring(2)
    r.issue(0, 0)
    r.wait_all()
    r.barrier()
    r.read(0, 0, wave=3)
    with pytest.raises(AssertionError):
        r.issue(0, 2)
    # reading a tile before the barrier that publishes it
    r = Ring(2)
    r.issue(1, 1)
    r.wait_all()
    with pytest.raises(AssertionError):
        r.read(1, 1, wave=0)
