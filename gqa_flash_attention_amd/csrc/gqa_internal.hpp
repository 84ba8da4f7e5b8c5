// gqa_internal.hpp - kernel argument blocks and launch entry points shared between the
// HIP kernel files and the C-ABI shim. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

struct PrefillArgs {
  const uint16_t* q;     // [B, S, Hq, D]
  const uint16_t* k;     // [B, S, Hkv, D]
  const uint16_t* v;     // [B, S, Hkv, D]
  uint16_t* out;         // [B, S, Hq, D]
  int B, S, Hq, Hkv, G;  // G = Hq / Hkv
  int nrb;               // 32-row query blocks per sequence: ceil(S / 32)
  int nw;                // (row block, head) units per workgroup (4 or 8; prefill_waves)
  int ks;                // key splits per unit (1, or 2 in the 4-unit form; prefill_key_splits)
  int wgs_per_slot;      // workgroups per (b, kv head): ceil(G * nrb / nw)
  int nslots;            // B * Hkv
  float c;               // scale * log2(e)
};

struct DecodeArgs {
  const uint16_t* q;     // [B, Hq, D]
  const uint16_t* kc;    // [B, L, Hkv, D]
  const uint16_t* vc;    // [B, L, Hkv, D]
  const int32_t* lens;   // [B], device
  float* o_part;         // [B, Hq, nsplit, D]
  float* lse;            // [B, Hq, nsplit], log2 units
  int* counters;         // [B, Hkv * hgroups] arrival counters of the fused merge (zero between calls)
  uint16_t* out;         // [B, Hq, D] (fused kernel only)
  int B, L, Hq, Hkv, G;
  int hgroups;           // ceil(G / 16): query heads are served 16 at a time
  int chunk;             // keys per split, a multiple of 64
  int nsplit;            // ceil(L / chunk)
  float c;               // scale * log2(e)
};

struct CombineArgs {
  const float* o_part;
  const float* lse;
  uint16_t* out;         // [B, Hq, D]
  int B, Hq, nsplit;
};

// Each returns a hipError_t value (0 = success) from the launch.
// Units (one wave each per key split) per prefill workgroup for this shape (4 or 8), and
// the key splits of the 4-unit form (1 or 2); a workgroup has nw * ks waves.
int prefill_waves(int B, int S, int Hkv, int G);
int prefill_key_splits(int B, int S, int Hkv, int G);
int launch_prefill(const PrefillArgs& a, bool causal, hipStream_t stream);
// The prefill with another tile shape (the sweep's forms other than the 64-key, 32-row
// ones): (rows_per_wave, keys_per_tile, waves) in {(32, 32, 4), (32, 32, 8), (32, 128, 4),
// (32, 128, 8), (64, 32, 4), (64, 64, 4)}; a.nw must be waves * rows_per_wave / 32.
int launch_prefill_tiles(const PrefillArgs& a, bool causal, int rows_per_wave, int keys_per_tile, int waves,
                         hipStream_t stream);
// fused = true: split, then merge in the last-arriving workgroup, writing `out`.
// fused = false: only the per-chunk partials (o_part, lse).
int launch_decode(const DecodeArgs& a, bool fused, hipStream_t stream);
int launch_decode_combine(const CombineArgs& a, hipStream_t stream);
// Fills n 32-bit words at p (device memory) with `value` on `stream` (a kernel, not a
// memset, so that the call may be captured into a HIP graph).
int launch_fill_words(uint32_t* p, size_t n, uint32_t value, hipStream_t stream);

// Measurement probes (probes.hip).
int launch_probe_hbm_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream);
int launch_probe_mfma_bf16(int rounds, uint32_t seed, int workgroups, float* sink, uint64_t* ticks,
                           hipStream_t stream);

// Rows per staged K/V tile (gqa_device.hpp's kTileRows) and bytes per bf16 row of
// D = 128, for the host-side bounds on tile offsets.
constexpr int kTileRowsHost = 64;
constexpr int kRowBytesHost = 128 * 2;

// Keys per split chosen for a decode of this shape (a multiple of 64).
int decode_default_chunk(int B, int L, int Hkv, int G);
// Largest accepted keys per split.
constexpr int kMaxChunk = 1 << 24;
// Most splits per sequence: the partials of one (sequence, KV head), up to 16 heads x
// nsplit x 512 B, then span at most 2 GiB and are addressed with 32-bit byte offsets.
constexpr int kMaxSplits = 1 << 18;

}  // namespace gqa
