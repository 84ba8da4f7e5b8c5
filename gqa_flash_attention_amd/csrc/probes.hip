// probes.hip - measured roofline denominators for the two kernels of the library.
//
// The metakernel page ("How it works") builds its device dossier from dedicated probe
// kernels rather than spec sheets: a read-only streaming kernel for DRAM bandwidth and a
// register-resident matrix-instruction loop per data type, each reported with the clock
// it ran at ("Return schemas": value, units, method, clock). These are the two probes the
// attention kernels need on gfx950:
//  - hbm_read: every byte of a caller buffer read once with 16-byte non-temporal loads,
//    the decode kernel's access width and cache policy (on MI355X non-temporal reads of
//    a 2 GiB buffer run ~6.0 TB/s against ~5.4 for plain ones). On a buffer several times
//    the 256 MB MALL this is the cold HBM read rate a decode can reach. When the buffer
//    is whole 2 KB rows and the workgroups a multiple of 8, the workgroups with id = x
//    (mod 8) read the 256-byte blocks at offset 256x of every row: the decode's pattern,
//    in which the workgroups of one XCD read one KV head's 256-byte slice of each cache
//    row (with round-robin dispatch, id mod 8 is the XCD). On MI355X that pattern reads a
//    2 GiB buffer at ~6.6-6.8 TB/s with 512 workgroups (2 per CU, long streams per lane;
//    ~6.2 with 1024-8192, 5.75 with 32768), ~5% faster than a plain grid-stride sweep.
//  - mfma_bf16: v_mfma_f32_32x32x16_bf16 from registers, 2 waves per SIMD on every CU, 8
//    independent accumulators per wave, the A and B operands drawn from 8 registers of
//    random bf16 each in a rotating pairing, so that consecutive instructions see new
//    data, as in attention. One round is 64 MFMAs per wave. Each
//    workgroup records shader-clock ticks (s_memtime) and 100 MHz ticks (s_memrealtime)
//    around its loop, so the clock the matrix cores actually ran at is measured too.
#include "gqa_device.hpp"
#include "gqa_internal.hpp"

namespace gqa {

namespace {

// An integer hash for the probe's random operands: the "lowbias32" xorshift-multiply
// function found by Chris Wellons' hash-prospector search (two multiply constants
// 0x7feb352d and 0x846ca68b, shifts 16/15/16), reimplemented here.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
  return x;
}

// A bf16 with random sign and mantissa and an exponent in [2^-3, 2^0]: roughly the spread
// of N(0, 1) activations.
__device__ __forceinline__ __bf16 random_bf16(uint32_t key) {
  const uint32_t r = mix32(key);
  const uint16_t bits = (uint16_t)((r & 0x8000U) | ((0x7CU + ((r >> 16) & 3U)) << 7) | (r & 0x7FU));
  return __builtin_bit_cast(__bf16, bits);
}

__global__ __launch_bounds__(256) void probe_hbm_read_kernel(const u32x4* src, size_t n16, uint32_t* sink,
                                                             int xcd_blocks) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  if (xcd_blocks) {
    // n16 = 128 * rows, gridDim.x = 8 * K. Workgroup (x = id mod 8, k = id / 8) reads block
    // x (16 chunks of 16 B) of rows 16 (k + K j) + t / 16, lane t taking chunk t mod 16.
    const size_t rows = n16 / 128;
    const size_t x = blockIdx.x & 7, k = blockIdx.x >> 3, K = gridDim.x >> 3;
    const size_t step = 16 * K;
    const size_t c = (size_t)(threadIdx.x & 15) + 16 * x;
    size_t r = 16 * k + (threadIdx.x >> 4);
    for (; r + 3 * step < rows; r += 4 * step) {
      const u32x4 a = __builtin_nontemporal_load(src + r * 128 + c);
      const u32x4 b = __builtin_nontemporal_load(src + (r + step) * 128 + c);
      const u32x4 d = __builtin_nontemporal_load(src + (r + 2 * step) * 128 + c);
      const u32x4 e = __builtin_nontemporal_load(src + (r + 3 * step) * 128 + c);
      acc ^= a ^ b ^ d ^ e;
    }
    for (; r < rows; r += step) acc ^= __builtin_nontemporal_load(src + r * 128 + c);
    sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    return;
  }
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = tid;
  // four independent 16-byte loads in flight per lane
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void probe_mfma_bf16_kernel(int rounds, uint32_t seed, float* sink, uint64_t* ticks) {
  bf16x8 av[8], bv[8];
  const uint32_t base = seed * 0x9E3779B9U + (uint32_t)(blockIdx.x * 256 + threadIdx.x) * 131U;
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      av[r][e] = random_bf16(base + 16 * r + e);
      bv[r][e] = random_bf16(base + 16 * r + e + 0x5bd1e995U);
    }
  f32x16 acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = f32x16{};
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < rounds; ++it) {
    // one round = 64 MFMAs per wave: step k multiplies A operand r with B operand (r+k)%8
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = mfma32(av[r], bv[(r + k) & 7], acc[r]);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[r][v];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    ticks[2 * blockIdx.x] = t1 - t0;
    ticks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

int launch_probe_hbm_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream) {
  const int xcd_blocks = (workgroups % 8 == 0 && bytes % 2048 == 0) ? 1 : 0;
  hipLaunchKernelGGL(probe_hbm_read_kernel, dim3(workgroups), dim3(256), 0, stream,
                     (const u32x4*)src, bytes / 16, sink, xcd_blocks);
  return (int)hipGetLastError();
}

int launch_probe_mfma_bf16(int rounds, uint32_t seed, int workgroups, float* sink, uint64_t* ticks,
                           hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_bf16_kernel, dim3(workgroups), dim3(256), 0, stream, rounds, seed, sink, ticks);
  return (int)hipGetLastError();
}

}  // namespace gqa
