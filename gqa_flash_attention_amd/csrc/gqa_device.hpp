// gqa_device.hpp - device-side building blocks shared by the prefill and decode kernels.
//
// Target: CDNA4 (gfx950), wave64. Everything here is written for that ISA:
//  - v_mfma_f32_32x32x16_bf16 / v_mfma_f32_16x16x32_bf16 (bf16 in, fp32 accumulate);
//  - global_load_lds_dwordx4: 16 B per lane straight from HBM into LDS;
//  - ds_read_b64_tr_b16: a transposing LDS read that hands each lane one column
//    of a 4x16 block of 16-bit values;
//  - v_permlane32_swap for exchanges between the two halves of a wave;
//  - v_exp_f32 (a native 2^x) for the softmax.
//
// Lane layouts (verified on the device with a one-wave probe):
//  32x32x16 MFMA: A[i][k] in lane i + 32*(k/8), element k%8; B[k][j] in lane
//    j + 32*(k/8), element k%8; D[i][j] in lane j + 32*((i/4)%2), element
//    4*(i/8) + i%4.
//  16x16x32 MFMA: A[i][k] in lane i + 16*(k/8); B[k][j] in lane j + 16*(k/8);
//    D[i][j] in lane j + 16*(i/4), element i%4.
//  ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
//    i%4 of the 8 bytes addressed by lane 4*e + i/4, as its element e (e=0..3).
//    With lane t addressing row t/4, column 4*(t%4) of a row-major 4x16 block,
//    lane i receives column i, rows 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define GQA_LDS __attribute__((address_space(3)))

constexpr int kD = 128;              // head dimension (the only one supported)
constexpr int kTileRows = 64;        // keys per staged K or V tile
constexpr int kRowBytes = kD * 2;    // one bf16 row: 256 B = 16 chunks of 16 B
constexpr int kTileBytes = kTileRows * kRowBytes;   // 16 KB

// ----------------------------------------------------------------------------------------
// LDS tile format. A tile holds 64 rows of 128 bf16. Row r occupies bytes [256r, 256r+256).
// Its 16-byte chunk c is stored at slot (c ^ swz(r)). The two swizzles are chosen so the
// two read patterns used below touch distinct LDS banks:
//  - K tiles are read as MFMA A operands: 16 (or 32) consecutive rows at one chunk. With
//    swz = r % 16, any 16 aligned consecutive rows land on 16 distinct slots.
//  - V tiles are read with ds_read_b64_tr_b16: 4 aligned consecutive rows x 2 or 4
//    chunks. With swz = f(r % 4), f = {0, 6, 10, 12}, both (f >> 1) % 4 and (f >> 2) % 4
//    are distinct over the 4 rows, so each 16-lane group reads 128 distinct bytes and
//    each 32-lane half reads 256 distinct bytes.
// ----------------------------------------------------------------------------------------
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return ((r & 1) ? 6 : 0) ^ ((r & 2) ? 10 : 0); }

// One 16-byte-per-lane copy from HBM straight into LDS (global_load_lds_dwordx4): lane j
// of the wave writes bytes [16j, 16j+16) after the wave-uniform LDS address `lds`.
// Issued through inline assembly on purpose: the compiler's wait-count pass cannot tell
// which LDS buffer such a copy writes, and when it sees one in flight it makes every
// later LDS read wait for all outstanding copies, including the prefetch of the next
// tile. Vector-memory loads complete in issue order, so the waits the compiler derives
// for its own loads stay conservative; the tile pipelines wait for these copies
// themselves (wait_vmcnt) before the barrier that publishes a tile.
// The LDS address travels in M0, passed as an operand so the compiler sets (and owns)
// M0; the leading s_nop covers the M0-write hazard before the copy reads it.
// NT marks the copy non-temporal (`nt`): data read once, such as a decode's KV cache,
// then does not displace what the caches hold (8% faster for a 64K-key decode on
// MI355X); data read again, such as the prefill's K/V tiles, must not use it (5-8%
// slower there).
template <bool NT = false>
__device__ __forceinline__ void lds_dma16(const void* gptr, GQA_LDS void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;
  if (NT) asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(gptr), "{m0}"(m0) : "memory");
  else    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "{m0}"(m0) : "memory");
}

// Same copy with the global address split into a wave-uniform 64-bit base (SGPRs) and a
// 32-bit per-lane byte offset (the saddr form): no per-lane 64-bit address arithmetic.
template <bool NT = false>
__device__ __forceinline__ void lds_dma16_sv(const void* sbase, uint32_t voff, GQA_LDS void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;
  if (NT) asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
  else    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// Per-lane byte offsets of a full 64-row K tile and V tile, computed once per kernel:
// the copy of any full tile is then just (tile base, offset) per instruction.
template <int NW, bool NT = false>
struct TileCopy {
  static constexpr int kPer = (kTileRows / 4) / NW;   // instructions per wave per tile
  uint32_t ko[kPer], vo[kPer];
  __device__ __forceinline__ void init(size_t row_stride_elems, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int r = 4 * (wave + NW * j) + (lane >> 4);
      const int slot = lane & 15;
      const uint32_t row = (uint32_t)(r * row_stride_elems * 2);
      ko[j] = row + (uint32_t)((slot ^ swz_k(r)) << 4);
      vo[j] = row + (uint32_t)((slot ^ swz_v(r)) << 4);
    }
  }
  // All 64 rows valid: K then V, kPer copies each for this wave.
  __device__ __forceinline__ void issue_full(GQA_LDS uint8_t* kt, GQA_LDS uint8_t* vt,
                                             const uint16_t* kg, const uint16_t* vg, int wave) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) lds_dma16_sv<NT>(kg, ko[j], kt + (wave + NW * j) * 1024);
#pragma unroll
    for (int j = 0; j < kPer; ++j) lds_dma16_sv<NT>(vg, vo[j], vt + (wave + NW * j) * 1024);
  }
};

// Issue the HBM->LDS copies of one 64-row tile. `rows` points at row 0 of the tile's
// head in global memory; consecutive rows are `row_stride` bf16 apart. Rows at or past
// `nvalid` (relative to the tile) are replaced by row nvalid-1, so every address read is
// a real row of the tensor (nvalid >= 1). Each wave instruction fills 1 KB = 4 rows; the
// NW waves of the workgroup take turns. Lane j of the instruction for rows 4i..4i+3
// writes LDS slot j of that 1 KB and fetches the global chunk that belongs there.
template <int NW, bool VTILE, bool NT = false>
__device__ __forceinline__ void stage_tile(GQA_LDS uint8_t* tile, const uint16_t* rows,
                                           size_t row_stride, int nvalid, int wave, int lane) {
#pragma unroll
  for (int i = wave; i < kTileRows / 4; i += NW) {
    const int r = 4 * i + (lane >> 4);
    const int slot = lane & 15;
    const int c = slot ^ (VTILE ? swz_v(r) : swz_k(r));
    const int gr = r < nvalid ? r : nvalid - 1;
    const uint16_t* src = rows + (size_t)gr * row_stride + c * 8;
    lds_dma16<NT>(src, tile + i * 1024);
  }
}

// 16-byte read of row r, chunk c of a K-format tile.
__device__ __forceinline__ bf16x8 lds_read_k(const GQA_LDS uint8_t* tile, int r, int c) {
  const GQA_LDS bf16x8* p = (const GQA_LDS bf16x8*)(tile + r * kRowBytes + ((c ^ swz_k(r)) << 4));
  return *p;
}

// Transposing read from a V-format tile. The calling lane names row r and the 4 columns
// starting at col (a multiple of 4). Returns 4 bf16 values as raw bits (see header note).
__device__ __forceinline__ s16x4 lds_read_v_tr(const GQA_LDS uint8_t* tile, int r, int col) {
  const int c = col >> 3;
  const int byte = r * kRowBytes + ((c ^ swz_v(r)) << 4) + ((col & 4) << 1);
  typedef GQA_LDS s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + byte));
}

__device__ __forceinline__ bf16x8 join_bf16x8(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Exchange between the two 32-lane halves of a wave: returns {x[l % 32], x[l % 32 + 32]}.
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
// IEEE 754-2019 maximum (v_maximum3_f32 on gfx950): unlike fmaxf it needs no quieting of
// its operands first, which the compiler otherwise emits as extra v_max_f32 x, x, x. NaN
// operands propagate; -inf (masked scores, an empty running max) behaves as in fmaxf.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float halves_max(float x) {
  float a, b;
  halves(x, a, b);
  return vmax(a, b);
}
__device__ __forceinline__ float halves_sum(float x) {
  float a, b;
  halves(x, a, b);
  return a + b;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even fp32 -> bf16 of 8 values (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
  bf16x8 r = {(__bf16)a0, (__bf16)a1, (__bf16)a2, (__bf16)a3,
              (__bf16)a4, (__bf16)a5, (__bf16)a6, (__bf16)a7};
  return r;
}

// Sum of the 8 bf16 values of v, accumulated into acc in fp32 (v_dot2_f32_bf16 against 1s).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[0], v[1]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2], v[3]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[4], v[5]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[6], v[7]}, one, acc, false);
  return acc;
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Workgroup execution barrier for the tile pipelines. Unlike __syncthreads() it carries
// no release/acquire fence, which would make every wave wait for all of its outstanding
// HBM->LDS copies (including the prefetch of the next tile) before the barrier. The
// callers wait for exactly the copies they need with wait_vmcnt<N>() first. The empty
// asm statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace gqa
