// decode.hip - one-token GQA decode against a KV cache on gfx950 (kernels K2 and K3).
//
// Implements the decode mode of the chowfi/kernels README ("Result": generate one token
// from a KV cache of a given length) with the two decode ideas of its "What helped
// most" section, redone for CDNA4:
//  - item 1 (split-KV): the cache is cut into chunks of `chunk` keys; one workgroup per
//    (chunk, KV head, sequence) spreads a single query over all 256 CUs (K2), and a
//    second kernel merges the chunks by log-sum-exp (K3);
//  - item 2 (GQA packing): a K2 workgroup reads each K/V row of its chunk once and
//    scores it against all query heads of the group (up to 16 per pass) with one
//    matrix-core instruction.
//
// K2 staging: every K/V tile of the chunk (64 rows each) is requested at the start with
// global_load_lds_dwordx4, so up to 256 rows x 512 B are in flight per workgroup with
// no register cost, and the chunk's first tiles are computed while later ones arrive.
// Rows at or past lens[b] are never requested: their addresses are redirected to the
// last valid row.
//
// K2 arithmetic, per wave and 32-key slab: S^T (16 keys x 16 heads, 4 heads real for
// Llama-3-8B) = K Q^T with v_mfma_f32_16x16x32_bf16 (K from LDS as the A operand, the
// query heads in registers as B); online softmax in base 2 per head; O^T (d x heads) +=
// V^T P^T, with V^T read by ds_read_b64_tr_b16 and P^T taken from the score accumulator
// as is. The waves of the workgroup then merge their (max, sum, O) through LDS, and the
// workgroup writes the chunk's normalised partial O (fp32) and its log-sum-exp (log2
// units). Matrix cores keep the arithmetic at a few percent of the HBM time.
#include "gqa_device.hpp"
#include "gqa_internal.hpp"

namespace gqa {

template <int T>
struct DecodeShape {
  static constexpr int NW = T == 1 ? 2 : 4;          // waves per workgroup
  static constexpr int kSlabs = 2 * T;               // 32-key slabs per chunk
  static constexpr int kLoadsPerTile = 2 * (16 / NW);  // K and V copies per wave per tile
};

template <int T, int N>
__device__ __forceinline__ void wait_tile() {
  wait_vmcnt<(T - 1 - N) * DecodeShape<T>::kLoadsPerTile>();
}

template <int T>
__global__ __launch_bounds__(DecodeShape<T>::NW * 64) void decode_split_kernel(DecodeArgs a) {
  constexpr int NW = DecodeShape<T>::NW;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[T * 2 * kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_q[16 * kRowBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x;
  const int g = blockIdx.y / a.hgroups;
  const int hg = blockIdx.y % a.hgroups;
  const int b = blockIdx.z;

  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.L ? a.L : len);
  const int key_begin = split * a.chunk;
  const int nkeys = min(a.chunk, len - key_begin);
  const int hbase = 16 * hg;                       // first head (within the group) served
  const int nheads = min(16, a.G - hbase);         // heads served by this workgroup
  float* lse_out = a.lse + ((size_t)b * a.Hq + g * a.G + hbase) * a.nsplit + split;
  if (nkeys <= 0) {
    // Nothing to attend in this chunk: weight zero in the merge.
    if (threadIdx.x < nheads) lse_out[(size_t)threadIdx.x * a.nsplit] = -INFINITY;
    return;
  }

  // Wave 0 first copies the served query heads (256 B each, 4 per instruction) into LDS,
  // then every wave issues its share of all K/V tiles. Every load of the kernel goes
  // through lds_dma16, so the per-tile waits below account for all of them; wave 0's
  // query copies are older than its tile copies and are covered by the first wait.
  const int n = lane & 15;
  const int grp = lane >> 4;
  if (wave == 0) {
    const uint16_t* qrow = a.q + ((size_t)b * a.Hq + g * a.G + hbase) * kD;
    for (int i = 0; 4 * i < nheads; ++i) {
      const int hh = min(4 * i + (lane >> 4), nheads - 1);
      lds_dma16(qrow + (size_t)hh * kD + 8 * (lane & 15), (GQA_LDS uint8_t*)lds_q + i * 1024);
    }
  }
  const size_t kv_stride = (size_t)a.Hkv * kD;
  const size_t row0 = ((size_t)b * a.L + key_begin) * a.Hkv + g;
  const uint16_t* kbase = a.kc + row0 * kD;
  const uint16_t* vbase = a.vc + row0 * kD;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    GQA_LDS uint8_t* kt = (GQA_LDS uint8_t*)lds + (2 * t) * kTileBytes;
    GQA_LDS uint8_t* vt = (GQA_LDS uint8_t*)lds + (2 * t + 1) * kTileBytes;
    const int r0 = t * kTileRows;
    // Rows past the valid keys (tile-relative nvalid <= 0) all map to the chunk's last
    // valid row, which stays inside the sequence.
    const int nvalid = nkeys - r0;
    const size_t off = nvalid > 0 ? (size_t)r0 * kv_stride : (size_t)(nkeys - 1) * kv_stride;
    stage_tile<NW, false>(kt, kbase + off, kv_stride, nvalid > 0 ? nvalid : 1, wave, lane);
    stage_tile<NW, true>(vt, vbase + off, kv_stride, nvalid > 0 ? nvalid : 1, wave, lane);
  }

  const float c = a.c;
  float m_run = -INFINITY;
  float l_part = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) oacc[mb] = f32x4{};

  bf16x8 qreg[4];
  auto slab = [&](const GQA_LDS uint8_t* kt, const GQA_LDS uint8_t* vt, int r0, int key0) {
    // r0: first tile row of the slab; key0: its first key within the chunk.
    f32x4 s[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kk = lds_read_k(kt, r0 + 16 * blk + n, 4 * ks + grp);
        s[blk] = mfma16(kk, qreg[ks], s[blk]);
      }
    }
    // s[blk][v]: head n, key key0 + 16 blk + 4 grp + v.
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x = s[blk][v] * c;
        if (key0 + 16 * blk + 4 * grp + v >= nkeys) x = -INFINITY;
        s[blk][v] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == m_run) ? 1.f : exp2_fast(m_run - m_new);
    m_run = m_new;
    l_part *= alpha;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) oacc[mb] *= alpha;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int v = 0; v < 4; ++v) s[blk][v] = exp2_fast(s[blk][v] - m_new);
    const bf16x8 p = to_bf16x8(s[0][0], s[0][1], s[0][2], s[0][3], s[1][0], s[1][1], s[1][2], s[1][3]);
    l_part = sum_bf16x8(p, l_part);
    // A operand V^T for d-block mb: lane holds d = 16mb + n and keys 4grp+{0..3}, 16+4grp+{0..3}.
    const int vr = r0 + 4 * grp + (n >> 2);
    const int vc = 4 * (n & 3);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const s16x4 lo = lds_read_v_tr(vt, vr, 16 * mb + vc);
      const s16x4 hi = lds_read_v_tr(vt, vr + 16, 16 * mb + vc);
      oacc[mb] = mfma16(join_bf16x8(lo, hi), p, oacc[mb]);
    }
  };

  // Query heads as the B operand (head = lane % 16, d = 32ks + 8(lane/16) + 0..7); heads
  // past nheads are zero. Read from LDS once the first tile (and so the query) landed.
  auto load_q = [&]() {
    const GQA_LDS uint8_t* qs = (const GQA_LDS uint8_t*)lds_q;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 x = *(const GQA_LDS bf16x8*)(qs + min(n, nheads - 1) * kRowBytes + (4 * ks + grp) * 16);
      qreg[ks] = n < nheads ? x : bf16x8{};
    }
  };

  auto tile = [&](auto tn) {
    constexpr int t = decltype(tn)::value;
    wait_tile<T, t>();
    tile_barrier();
    if (t == 0) load_q();
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int sid = 2 * t + sl;
      if (sid % NW != wave) continue;
      const int key0 = sid * 32;
      if (key0 >= nkeys) continue;
      const GQA_LDS uint8_t* kt = (const GQA_LDS uint8_t*)lds + (2 * t) * kTileBytes;
      const GQA_LDS uint8_t* vt = (const GQA_LDS uint8_t*)lds + (2 * t + 1) * kTileBytes;
      slab(kt, vt, 32 * sl, key0);
    }
  };
  tile(std::integral_constant<int, 0>{});
  if constexpr (T > 1) tile(std::integral_constant<int, 1>{});
  if constexpr (T > 2) tile(std::integral_constant<int, 2>{});
  if constexpr (T > 3) tile(std::integral_constant<int, 3>{});

  // The 4 lane groups of a wave hold disjoint keys of the same heads.
  l_part += __shfl_xor(l_part, 16);
  l_part = halves_sum(l_part);

  // Merge the waves through LDS (the tiles are no longer needed).
  __syncthreads();
  GQA_LDS float* wo = (GQA_LDS float*)lds;       // [NW][16][128] per-wave O
  GQA_LDS float* wm = wo + NW * 16 * kD;         // [NW][16] per-wave max
  GQA_LDS float* wl = wm + NW * 16;              // [NW][16] per-wave sum
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) wo[(wave * 16 + n) * kD + 16 * mb + 4 * grp + v] = oacc[mb][v];
  if (grp == 0) {
    wm[wave * 16 + n] = m_run;
    wl[wave * 16 + n] = l_part;
  }
  __syncthreads();
  float* opart = a.o_part + (((size_t)b * a.Hq + g * a.G + hbase) * a.nsplit + split) * kD;
  for (int idx = threadIdx.x; idx < nheads * kD; idx += NW * 64) {
    const int hn = idx / kD;
    const int d = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w * 16 + hn]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = wm[w * 16 + hn];
      const float sc = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
      num += sc * wo[(w * 16 + hn) * kD + d];
      den += sc * wl[w * 16 + hn];
    }
    opart[(size_t)hn * a.nsplit * kD + d] = num / den;
    if (d == 0) lse_out[(size_t)hn * a.nsplit] = M + log2f(den);
  }
}

// K3: out[b, h, :] = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), M = max finite lse_s.
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
  const int hgroups = (G + 15) / 16;
  const long long wgs128 = (long long)B * Hkv * hgroups * ((L + 127) / 128);
  return wgs128 < 1024 ? 64 : 128;
}

int launch_decode_split(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.nsplit, (unsigned)(a.Hkv * a.hgroups), (unsigned)a.B);
  switch (a.chunk / kTileRows) {
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(DecodeShape<1>::NW * 64), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, dim3(DecodeShape<2>::NW * 64), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(decode_split_kernel<3>, grid, dim3(DecodeShape<3>::NW * 64), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(decode_split_kernel<4>, grid, dim3(DecodeShape<4>::NW * 64), 0, stream, a); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_decode_combine(const CombineArgs& a, hipStream_t stream) {
  const dim3 grid(kD / 32, (unsigned)a.Hq, (unsigned)a.B);
  hipLaunchKernelGGL(decode_combine_kernel, grid, dim3(256), 0, stream, a);
  return (int)hipGetLastError();
}

}  // namespace gqa
