// decode.hip - one-token GQA decode against a KV cache on gfx950.
//
// Implements the decode mode of the chowfi/kernels README ("Result": generate one token
// from a KV cache of a given length) with the decode ideas of its "What helped most"
// section, redone for CDNA4:
//  - item 1 (split-KV): the cache is cut into splits; one workgroup per (split, KV head,
//    sequence) spreads a single query over all 256 CUs, and the split results are merged
//    by log-sum-exp;
//  - item 2 (GQA packing): a workgroup reads each K/V row of its split once and scores it
//    against all query heads of the group (up to 16 per pass) with one matrix-core
//    instruction;
//  - item 5 (one fewer launch in short decodes): the merge is fused into the same kernel.
//    The last workgroup of a (sequence, KV head) to finish merges the partials of all
//    splits; with a single split the result is written directly.
//
// Streaming. A workgroup walks its split's keys in 64-key tiles through an LDS ring of
// NSTAGE stages (K 16 KB + V 16 KB each). Tiles are copied with global_load_lds_dwordx4
// straight from HBM into LDS, NSTAGE-1 tiles ahead, so ~96 KB per CU stay in flight with
// no register cost. The copies are issued by eight waves, of which four also attend and
// four only copy (and leave once the last tile has landed): with twice the waves issuing
// loads a CU keeps more of them in flight (paired on MI355X: 0.3-0.9 us faster at 16K-64K
// keys; a pure cold read of the same pattern gains ~10% from 4 to 8 waves per CU). Rows at
// or past lens[b] are never requested: their addresses are redirected to the last valid row. The library sizes splits so that a batch-1 decode is
// about one workgroup per CU. Which tiles a split holds depends on the entry point:
//  - the stand-alone partials: split s is the chunk [s*chunk, (s+1)*chunk), walked from
//    its tile 5s (mod its tile count) round, so that the reads in flight at one moment
//    are not all at one offset into slabs a chunk apart (~4% slower on MI355X for a
//    pure-read kernel of the batch-1, 64K-key shape). Only the summation order changes;
//  - the fused decode, whose partials never leave the kernel: split s takes tiles s,
//    s + nsplit, s + 2 nsplit, ... of the whole sequence, so at any moment the
//    workgroups of a head read one contiguous stretch of the cache (a further 1-4% for
//    the same pure-read kernel at 16K-64K keys), and a short sequence in a batch spreads
//    over all its splits instead of leaving the last ones empty.
//
// Arithmetic per wave (16 keys of each tile): S^T (16 keys x 16 heads; 4 heads are real
// for Llama-3-8B) = K Q^T with v_mfma_f32_16x16x32_bf16, K from LDS as the A operand and
// the query heads in registers as B; an online softmax in base 2 per head; then
// O^T (d x heads) += V^T P^T with v_mfma_f32_16x16x16_bf16, whose B operand is the score
// accumulator layout as is and whose A operand (V^T) comes from ds_read_b64_tr_b16.
// The four waves merge their (max, sum, O) through LDS at the end of the split.
#include "gqa_device.hpp"
#include "gqa_internal.hpp"

namespace gqa {

constexpr int kDecWaves = 4;       // waves that attend
constexpr int kDecCopyWaves = 8;   // waves that issue the tile copies (the extra 4 only copy)
constexpr int kDecLoadsPerTile = 2 * (kTileRows / 4) / kDecCopyWaves;   // K and V copies per wave per tile

__device__ __forceinline__ f32x4 mfma16k16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// wait until at most `ahead` tiles of this wave's copies are still in flight
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  switch (ahead) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<kDecLoadsPerTile>(); break;
    case 2: wait_vmcnt<2 * kDecLoadsPerTile>(); break;
    default: wait_vmcnt<3 * kDecLoadsPerTile>(); break;
  }
}

// Partials cross workgroups (and XCDs, each with its own L2): they are written with
// device-coherent stores (relaxed atomic stores at agent scope, sc1) and read back by the
// merging workgroup with device-coherent loads, so no fence has to write back or
// invalidate a whole cache.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-coherent 16-byte load and store: buffer accesses with the agent-scope coherence
// bit (sc1), the encoding of relaxed agent-scope atomic loads and stores. Offsets past
// the resource's size read zero and are not written.
constexpr int kBufferDword3 = 0x00020000;   // raw 32-bit buffer resource word 3 on gfx9
constexpr int kCachePolicySC1 = 16;
__device__ __forceinline__ f32x4 load_coherent16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kCachePolicySC1));
}
__device__ __forceinline__ void store_coherent16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)byte_off, 0, kCachePolicySC1);
}

// FUSE: merge the splits in the last-arriving workgroup (and write bf16 out); otherwise
// only write the per-split partials. STRIDED: the tile-to-split assignment of the fused
// decode (see the top of this file); otherwise contiguous chunks.
template <int NSTAGE, bool FUSE, bool STRIDED>
__global__ __launch_bounds__(512) void decode_kernel(DecodeArgs a) {
  static_assert(NSTAGE >= 2 && NSTAGE <= 5, "ring depth");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * 2 * kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_q[16 * kRowBytes];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;      // query head (within the served group) of this lane
  const int grp = lane >> 4;    // which 4 of the wave's 16 keys this lane scores
  // Workgroups are numbered with the (KV head, head group) slot fastest: with round-robin
  // dispatch over the 8 XCDs and 8 KV heads, each XCD then streams one KV head (3.5%
  // faster at 64K keys on MI355X than interleaving the heads over the XCDs).
  const int hgs = a.Hkv * a.hgroups;
  const int split = (int)(blockIdx.x / hgs);
  const int gy = (int)(blockIdx.x % hgs);
  const int g = gy / a.hgroups;
  const int hg = gy % a.hgroups;
  const int b = blockIdx.z;

  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.L ? a.L : len);
  int ntiles, rot = 0;
  if (STRIDED) {
    const int T = (len + kTileRows - 1) / kTileRows;   // tiles of the sequence
    ntiles = split < T ? (T - 1 - split) / a.nsplit + 1 : 0;
  } else {
    const int nkeys = min(a.chunk, len - split * a.chunk);
    ntiles = nkeys > 0 ? (nkeys + kTileRows - 1) / kTileRows : 0;
    rot = ntiles > 0 ? (5 * split) % ntiles : 0;
  }
  // First key (counted from the start of the sequence) of the t-th tile this workgroup
  // streams. Chunks are whole tiles, so the only partial tile is the one holding key
  // len - 1, and a tile starting at key k holds min(64, len - k) keys.
  auto tile_key = [&](int t) {
    if (STRIDED) return (t * a.nsplit + split) * kTileRows;
    const int p = t + rot < ntiles ? t + rot : t + rot - ntiles;
    return split * a.chunk + p * kTileRows;
  };
  const int hbase = 16 * hg;
  const int nheads = min(16, a.G - hbase);
  const size_t head0 = (size_t)b * a.Hq + (size_t)g * a.G + hbase;   // first served head row
  float* lse_out = a.lse + head0 * a.nsplit + split;
  // o_part rows of the served heads: [nheads][nsplit][kD] fp32
  const __amdgpu_buffer_rsrc_t o_rows = __builtin_amdgcn_make_buffer_rsrc(
      a.o_part + head0 * a.nsplit * kD, (short)0, (int)((uint32_t)nheads * (uint32_t)a.nsplit * (kD * 4u)),
      kBufferDword3);

  if (ntiles > 0) {
    const size_t kv_stride = (size_t)a.Hkv * kD;
    const size_t row0 = (size_t)b * a.L * a.Hkv + g;
    const uint16_t* kbase = a.kc + row0 * kD;
    const uint16_t* vbase = a.vc + row0 * kD;
    GQA_LDS uint8_t* const ring = (GQA_LDS uint8_t*)lds;

    // Wave 0 first copies the served query heads (256 B each, 4 heads per instruction);
    // they are the oldest copies in flight, so the first tile wait covers them.
    if (wave == 0) {
      const uint16_t* qrow = a.q + head0 * kD;
      for (int i = 0; 4 * i < nheads; ++i) {
        const int hh = min(4 * i + (lane >> 4), nheads - 1);
        lds_dma16(qrow + (size_t)hh * kD + 8 * (lane & 15), (GQA_LDS uint8_t*)lds_q + i * 1024);
      }
    }
    TileCopy<kDecCopyWaves, true> copy;   // the cache is read once: non-temporal copies
    copy.init(kv_stride, wave, lane);
    // Copies of the t-th streamed tile (K then V): per-lane offsets for a full tile, the
    // clamped per-row path for the ragged last tile.
    auto issue = [&](int t) {
      GQA_LDS uint8_t* st = ring + (t % NSTAGE) * (2 * kTileBytes);
      const int r0 = tile_key(t);
      const size_t off = (size_t)r0 * kv_stride;
      if (len - r0 >= kTileRows) {
        copy.issue_full(st, st + kTileBytes, kbase + off, vbase + off, wave);
      } else {
        stage_tile<kDecCopyWaves, false, true>(st, kbase + off, kv_stride, len - r0, wave, lane);
        stage_tile<kDecCopyWaves, true, true>(st + kTileBytes, vbase + off, kv_stride, len - r0, wave, lane);
      }
    };
    for (int t = 0; t < NSTAGE - 1; ++t)
      if (t < ntiles) issue(t);

    const float c = a.c;
    float m_run = -INFINITY;
    float l_part = 0.f;
    f32x4 oacc[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) oacc[mb] = f32x4{};
    bf16x8 qreg[4];

    for (int t = 0; t < ntiles; ++t) {
      wait_tiles_ahead(min(NSTAGE - 2, ntiles - 1 - t));
      // Tile t is in LDS for every wave, and every wave is done with tile t-1, whose
      // stage the copy below refills.
      tile_barrier();
      if (t == 0) {
        const GQA_LDS uint8_t* qs = (const GQA_LDS uint8_t*)lds_q;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 x = *(const GQA_LDS bf16x8*)(qs + min(n, nheads - 1) * kRowBytes + (4 * ks + grp) * 16);
          qreg[ks] = n < nheads ? x : bf16x8{};
        }
      }
      if (t + NSTAGE - 1 < ntiles) issue(t + NSTAGE - 1);

      const int kw = tile_key(t) + 16 * wave;   // first key of this wave
      if (wave < kDecWaves && kw < len) {
        const GQA_LDS uint8_t* kt = ring + (t % NSTAGE) * (2 * kTileBytes);
        const GQA_LDS uint8_t* vt = kt + kTileBytes;
        f32x4 s = f32x4{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          s = mfma16(lds_read_k(kt, 16 * wave + n, 4 * ks + grp), qreg[ks], s);
        // s[v]: head n, key kw + 4 grp + v
        float x[4];
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          x[v] = (kw + 4 * grp + v < len) ? s[v] * c : -INFINITY;
          mx = vmax(mx, x[v]);
        }
        mx = vmax(mx, __shfl_xor(mx, 16));
        mx = halves_max(mx);
        const float m_new = vmax(m_run, mx);
        const float alpha = (m_new == m_run) ? 1.f : exp2_fast(m_run - m_new);
        m_run = m_new;
        l_part *= alpha;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) oacc[mb] *= alpha;
        const __bf16 p0 = (__bf16)exp2_fast(x[0] - m_new), p1 = (__bf16)exp2_fast(x[1] - m_new);
        const __bf16 p2 = (__bf16)exp2_fast(x[2] - m_new), p3 = (__bf16)exp2_fast(x[3] - m_new);
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        l_part = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0, p1}, one, l_part, false);
        l_part = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p2, p3}, one, l_part, false);
        const s16x4 pb = {__builtin_bit_cast(short, p0), __builtin_bit_cast(short, p1),
                          __builtin_bit_cast(short, p2), __builtin_bit_cast(short, p3)};
        // A operand V^T for d-block mb: lane holds d = 16mb + n, keys kw + 4grp + 0..3.
        const int vr = 16 * wave + 4 * grp + (n >> 2);
        const int vc = 4 * (n & 3);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
          oacc[mb] = mfma16k16(lds_read_v_tr(vt, vr, 16 * mb + vc), pb, oacc[mb]);
      }
    }

    // The copy-only waves are done: their copies all landed before the last tile's
    // barrier. A barrier after this waits only for the waves still running.
    if (wave >= kDecWaves) return;
    // The 4 lane groups of a wave hold disjoint keys of the same heads.
    l_part += __shfl_xor(l_part, 16);
    l_part = halves_sum(l_part);

    // Merge the waves through LDS (every copy has landed: the last wait was vmcnt(0)).
    // Rows of 132 floats put the 16 lanes of a 16-byte write on distinct banks.
    __syncthreads();
    constexpr int kWo = kD + 4;
    GQA_LDS float* wo = (GQA_LDS float*)lds;       // [4][16][kWo] per-wave O, real heads only
    GQA_LDS float* wm = wo + kDecWaves * 16 * kWo; // [4][16] per-wave max
    GQA_LDS float* wl = wm + kDecWaves * 16;       // [4][16] per-wave sum
    if (n < nheads) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
        *(GQA_LDS f32x4*)(wo + (wave * 16 + n) * kWo + 16 * mb + 4 * grp) = oacc[mb];
      if (grp == 0) {
        wm[wave * 16 + n] = m_run;
        wl[wave * 16 + n] = l_part;
      }
    }
    __syncthreads();
    // thread -> (head, 4 consecutive d)
    for (int col = threadIdx.x; col < nheads * (kD / 4); col += 256) {
      const int hn = col / (kD / 4);
      const int d4 = 4 * (col % (kD / 4));
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, wm[w * 16 + hn]);
      f32x4 num = f32x4{};
      float den = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = wm[w * 16 + hn];
        const float sc = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
        num += sc * *(const GQA_LDS f32x4*)(wo + (w * 16 + hn) * kWo + d4);
        den += sc * wl[w * 16 + hn];
      }
      if (FUSE && a.nsplit == 1) {
        typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
        u16x4 o;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = bf16_bits(num[v] / den);
        *(u16x4*)(a.out + (head0 + hn) * kD + d4) = o;
      } else {
        f32x4 o;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = num[v] / den;
        store_coherent16(o_rows, (uint32_t)(((hn * a.nsplit + split) * kD + d4) * 4), o);
        if (d4 == 0) publish(lse_out + (size_t)hn * a.nsplit, M + log2f(den));
      }
    }
  } else {
    // Nothing to attend in this split: weight zero in the merge.
    if (wave >= kDecWaves) return;
    if (threadIdx.x < nheads) publish(lse_out + (size_t)threadIdx.x * a.nsplit, -INFINITY);
    if (FUSE && a.nsplit == 1) {
      for (int idx = threadIdx.x; idx < nheads * kD; idx += 256) a.out[head0 * kD + idx] = 0;
    }
  }

  if (!FUSE || a.nsplit == 1) return;

  // Count this split, in this order:
  //  1. each thread waits until its own partial stores have completed (vmcnt(0): a
  //     device-coherent store counts as completed once it is visible at agent scope);
  //  2. the barrier then tells thread 0 that every thread of the workgroup got there;
  //  3. only then does thread 0 count the split.
  // So when the last workgroup's count returns, every split's partial is in memory. That
  // workgroup merges them, reading with device-coherent loads (which cannot hit a stale
  // line in its XCD's L2, so no cache-wide invalidation is needed), and afterwards resets
  // the counter for the next call. No workgroup ever waits for another. The wait in 1 is
  // explicit, not left to how the barrier's own fence happens to be lowered.
  wait_vmcnt<0>();
  __syncthreads();
  int* counter = a.counters + (size_t)b * a.Hkv * a.hgroups + gy;
  if (threadIdx.x == 0)
    s_last = (__hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.nsplit - 1);
  __syncthreads();
  if (!s_last) return;

  // out[h, d] = sum_s 2^(lse_s - M) o_s[d] / sum_s 2^(lse_s - M). Thread -> (head, 4
  // consecutive d) column and a share of the splits, kBatch splits per round of loads;
  // within a round one maximum and independent weights, across rounds a rescale.
  constexpr int kBatch = 16;
  const int ncols = nheads * (kD / 4);
  const int nparts = ncols >= 256 ? 1 : 256 / ncols;
  GQA_LDS float* red = (GQA_LDS float*)lds;      // [nparts][ncols][6]
  const float* lse_all = a.lse + head0 * a.nsplit;
  for (int base = 0; base < ncols * nparts; base += 256) {
    const int u = base + threadIdx.x;
    const bool act = u < ncols * nparts;
    const int col = u % ncols;
    const int part = u / ncols;
    const int hn = col / (kD / 4);
    const int d4 = (col % (kD / 4)) * 4;
    float m = -INFINITY, den = 0.f;
    f32x4 num = f32x4{};
    if (act) {
      const float* lrow = lse_all + (size_t)hn * a.nsplit;
      const uint32_t orow = (uint32_t)((hn * a.nsplit * kD + d4) * 4);
      for (int s0 = part; s0 < a.nsplit; s0 += kBatch * nparts) {
        float lv[kBatch];
        f32x4 ov[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int s = min(s0 + j * nparts, a.nsplit - 1);
          lv[j] = __hip_atomic_load(lrow + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ov[j] = load_coherent16(o_rows, orow + (uint32_t)s * (kD * 4));
        }
        float mb = m;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          // past the last split, or an empty split (lse = -inf, o_part row never written)
          if (s0 + j * nparts >= a.nsplit || lv[j] == -INFINITY) {
            lv[j] = -INFINITY;
            ov[j] = f32x4{};
          }
          mb = fmaxf(mb, lv[j]);
        }
        if (mb == -INFINITY) continue;
        if (mb > m) {
          const float sc = exp2_fast(m - mb);   // 0 while nothing has been folded
          num *= sc;
          den *= sc;
          m = mb;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const float w = exp2_fast(lv[j] - m);
          num += w * ov[j];
          den += w;
        }
      }
    }
    if (nparts > 1) {
      __syncthreads();
      if (act) {
        GQA_LDS float* r = red + ((size_t)part * ncols + col) * 6;
        r[0] = m; r[1] = den; r[2] = num[0]; r[3] = num[1]; r[4] = num[2]; r[5] = num[3];
      }
      __syncthreads();
      if (act && part == 0) {
        for (int p = 1; p < nparts; ++p) {
          const GQA_LDS float* r = red + ((size_t)p * ncols + col) * 6;
          const float mp = r[0];
          if (mp == -INFINITY) continue;
          const float mn = fmaxf(m, mp);
          const float so = (m == -INFINITY) ? 0.f : exp2_fast(m - mn);
          const float sp = exp2_fast(mp - mn);
          den = den * so + r[1] * sp;
          num[0] = num[0] * so + r[2] * sp;
          num[1] = num[1] * so + r[3] * sp;
          num[2] = num[2] * so + r[4] * sp;
          num[3] = num[3] * so + r[5] * sp;
          m = mn;
        }
      }
    }
    if (act && part == 0) {
      typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
      const float inv = den > 0.f ? 1.f / den : 0.f;
      u16x4 w;
      w[0] = bf16_bits(num[0] * inv);
      w[1] = bf16_bits(num[1] * inv);
      w[2] = bf16_bits(num[2] * inv);
      w[3] = bf16_bits(num[3] * inv);
      *(u16x4*)(a.out + (head0 + hn) * kD + d4) = w;
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stand-alone merge of per-split partials (the second half of a decode on its own):
// out[b, h, :] = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), M = max finite lse_s.
// Grid (D/32, Hq, B); 256 threads = 8 groups of 32 lanes; lane -> d, group -> splits.
__global__ __launch_bounds__(256) void decode_combine_kernel(CombineArgs a) {
  __shared__ float red_m[8];
  __shared__ float red_num[8][32];
  __shared__ float red_den[8];
  const int lane = threadIdx.x & 31;
  const int grp = threadIdx.x >> 5;
  const int d = 32 * blockIdx.x + lane;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const size_t row = (size_t)b * a.Hq + h;
  const float* lse = a.lse + row * a.nsplit;
  const float* op = a.o_part + row * a.nsplit * kD;

  float M = -INFINITY;
  for (int s = threadIdx.x; s < a.nsplit; s += 256) M = fmaxf(M, lse[s]);
  for (int off = 16; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 32));
  if (lane == 0) red_m[grp] = M;
  __syncthreads();
  M = red_m[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) M = fmaxf(M, red_m[i]);

  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s = grp; s < a.nsplit; s += 8) {
      const float l = lse[s];
      if (l == -INFINITY) continue;
      const float w = exp2_fast(l - M);
      num += w * op[(size_t)s * kD + d];
      den += w;
    }
  }
  red_num[grp][lane] = num;
  if (lane == 0) red_den[grp] = den;
  __syncthreads();
  if (grp == 0) {
    float tn = 0.f, td = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) { tn += red_num[i][lane]; td += red_den[i]; }
    a.out[row * kD + d] = bf16_bits(td > 0.f ? tn / td : 0.f);
  }
}

int decode_default_chunk(int B, int L, int Hkv, int G) {
  // About one workgroup per CU (each (sequence, KV head) slot's cache cut into
  // L * slots / 256 keys per split), at least 128 keys and at most 4096 per split. Measured
  // on MI355X with the fused decode's strided splits: batch 1, L = 2K..64K: 128-key splits
  // are fastest at 2K, ~L/32 from 16K up; batched caches (B = 4..64, uniform or ragged
  // lengths up to 50001) run as fast or faster with 4096-key splits than with 1024 (up to
  // 11% at B = 64, L = 4K, and 10% for a ragged batch of 16). Splits of fewer than 8 tiles
  // are doubled while that still leaves at least 128 workgroups: at batch 1, 256-key splits
  // (128 workgroups) are 8% faster than 128-key ones (256 workgroups) at 4K keys and
  // 512-key ones 2% faster than 256 at 8K, while at 2K 256-key splits (64 workgroups) are
  // 3% slower than 128.
  const long long slots = (long long)B * Hkv * ((G + 15) / 16);
  const long long per = ((long long)L * slots + 255) / 256;
  long long chunk = (per + kTileRows - 1) / kTileRows * kTileRows;
  if (chunk < 2 * kTileRows) chunk = 2 * kTileRows;
  while (chunk < 8 * kTileRows && ((long long)L / (2 * chunk)) * slots >= 128) chunk *= 2;
  if (chunk > 4096) chunk = 4096;
  return (int)chunk;
}

int launch_decode(const DecodeArgs& a, bool fused, hipStream_t stream) {
  const dim3 grid((unsigned)(a.nsplit * a.Hkv * a.hgroups), 1, (unsigned)a.B);
  if (fused) hipLaunchKernelGGL((decode_kernel<4, true, true>), grid, dim3(512), 0, stream, a);
  else       hipLaunchKernelGGL((decode_kernel<4, false, false>), grid, dim3(512), 0, stream, a);
  return (int)hipGetLastError();
}

int launch_decode_combine(const CombineArgs& a, hipStream_t stream) {
  const dim3 grid(kD / 32, (unsigned)a.Hq, (unsigned)a.B);
  hipLaunchKernelGGL(decode_combine_kernel, grid, dim3(256), 0, stream, a);
  return (int)hipGetLastError();
}

// Fills a new workspace's merge counters (with zero). A kernel rather than
// hipMemsetAsync so that a caller may capture the first decode on a stream into a HIP graph.
__global__ __launch_bounds__(256) void fill_words_kernel(uint32_t* p, size_t n, uint32_t value) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = value;
}

int launch_fill_words(uint32_t* p, size_t n, uint32_t value, hipStream_t stream) {
  if (n == 0) return 0;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_words_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream, p, n,
                     value);
  return (int)hipGetLastError();
}

}  // namespace gqa
