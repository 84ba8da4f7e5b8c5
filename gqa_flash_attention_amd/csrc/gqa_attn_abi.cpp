// gqa_attn_abi.cpp - the C ABI of libgqa_attn.so: argument checks, split planning,
// workspace management and launches on the caller's stream. The declarations and the
// contract of every entry point are in include/gqa_attn.h.
#include "gqa_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "gqa_internal.hpp"

namespace {

thread_local std::string g_last_error;

int hip_fail(const char* what, int err) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), "%s: %s (%d)", what, hipGetErrorString((hipError_t)err), err);
  g_last_error = buf;
  return GQA_ATTN_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr double kLog2e = 1.4426950408889634;
constexpr long long kMaxGridY = 65535;

// Shared shape checks. Returns 0 or an error code.
int check_heads(int Hq, int Hkv, int D, float scale) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return GQA_ATTN_ERR_DIM;
  if (!std::isfinite(scale)) return GQA_ATTN_ERR_DIM;
  if (D != 128) return GQA_ATTN_ERR_UNSUPPORTED;
  return 0;
}

// Elements of a [n0, n1, n2, 128] tensor, or -1 if that overflows 2^62.
long long elems4(long long n0, long long n1, long long n2) {
  const long long lim = (1LL << 62) / 128;
  if (n0 > lim / n1) return -1;
  long long x = n0 * n1;
  if (x > lim / n2) return -1;
  return x * n2 * 128;
}

struct DecodeShapeCheck {
  int code;
  int chunk;
  int nsplit;
  int hgroups;
};

DecodeShapeCheck check_decode_shape(int B, int L, int Hq, int Hkv, int D, float scale, int chunk) {
  DecodeShapeCheck r{0, 0, 0, 0};
  if (B < 1 || L < 1) { r.code = GQA_ATTN_ERR_DIM; return r; }
  if ((r.code = check_heads(Hq, Hkv, D, scale)) != 0) return r;
  if (elems4(B, L, Hkv) < 0 || elems4(B, Hq, 1) < 0) { r.code = GQA_ATTN_ERR_DIM; return r; }
  const int G = Hq / Hkv;
  r.hgroups = (G + 15) / 16;
  if (B > kMaxGridY || (long long)Hkv * r.hgroups > kMaxGridY) { r.code = GQA_ATTN_ERR_DIM; return r; }
  if (chunk == 0) chunk = gqa::decode_default_chunk(B, L, Hkv, G);
  if (chunk < 64 || chunk % 64 != 0 || chunk > gqa::kMaxChunk) { r.code = GQA_ATTN_ERR_WORKSPACE; return r; }
  r.chunk = chunk;
  const long long nsplit = ((long long)L + chunk - 1) / chunk;
  if (nsplit > gqa::kMaxSplits) { r.code = GQA_ATTN_ERR_WORKSPACE; return r; }
  // the decode grid has nsplit * Hkv * hgroups workgroups in one dimension
  if (nsplit * Hkv * r.hgroups > 0x7fffffffLL) { r.code = GQA_ATTN_ERR_DIM; return r; }
  r.nsplit = (int)nsplit;
  if (elems4(B, Hq, r.nsplit) < 0) { r.code = GQA_ATTN_ERR_DIM; return r; }
  return r;
}

// Workspace layout, each part on a 256-byte boundary:
//   int32 counters[max(4096, B*Hq)] | fp32 o_part[B][Hq][nsplit][128] | fp32 lse[B][Hq][nsplit].
// The counters come first and their region depends only on (B, Hq), so a workspace
// reused for another shape finds its counters where the last call left them: zero.
// (B*Hq bounds the B*Hkv*ceil(G/16) counters a decode uses.)
struct WsLayout {
  size_t o_off, lse_off, cnt_count, total;
};
WsLayout ws_layout(int B, int Hq, int nsplit) {
  const size_t rows = (size_t)B * Hq * nsplit;
  WsLayout w;
  w.cnt_count = (size_t)B * Hq > 4096 ? (size_t)B * Hq : 4096;
  w.o_off = (w.cnt_count * sizeof(int) + 255) / 256 * 256;
  w.lse_off = w.o_off + (rows * 128 * sizeof(float) + 255) / 256 * 256;
  w.total = w.lse_off + (rows * sizeof(float) + 255) / 256 * 256;
  return w;
}
size_t ws_bytes_for(int B, int Hq, int nsplit) { return ws_layout(B, Hq, nsplit).total; }

// Library-owned decode workspaces, one per (device, stream), grown on demand. A buffer
// that has been handed to a launch is never freed before gqa_attn_release: when a larger
// one replaces it, it moves to the retired list, because earlier launches on the stream,
// or a HIP graph captured from one, may still use it.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, void*>, Workspace> g_ws;
std::vector<std::pair<int, void*>> g_retired;   // (device, buffer)

// With g_ws_mutex held by the caller (until its launch has been enqueued, so that no
// other thread can retire the buffer in between).
int get_workspace(size_t need, hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  Workspace& w = g_ws[{dev, (void*)stream}];
  if (w.bytes < need) {
    const size_t grow = (need + (1u << 20) - 1) / (1u << 20) * (1u << 20);
    void* p = nullptr;
    e = hipMalloc(&p, grow);
    if (e != hipSuccess) return hip_fail("hipMalloc(decode workspace)", e);
    // The merge counters must start at zero (every completed decode leaves them zero):
    // cleared on the stream, ahead of the launch that will use the buffer.
    const int fe = gqa::launch_fill_words((uint32_t*)p, grow / 4, 0u, stream);
    if (fe != 0) {
      (void)hipFree(p);
      return hip_fail("fill_words launch (decode workspace)", fe);
    }
    if (w.ptr) g_retired.emplace_back(dev, w.ptr);
    w.ptr = p;
    w.bytes = grow;
  }
  *out = w.ptr;
  return 0;
}

// Scratch for gqa_attn_decode_noalloc: the decode workspace of callers that cannot
// allocate. One copy per GPU (a device global lives on every device the library runs on),
// kept until the process ends. Host code never uses the array's name as an address: the
// per-device address comes from hipGetSymbolAddress (scratch_on_current_device).
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The device address of `scratch` per device ordinal, looked up once; a fixed table, so that
// the entry point allocates no host memory either.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// With g_scratch_mutex held: the address of the current device's scratch. The first call on
// a device looks the address up and clears the whole array (a kernel on `stream`, so the
// merge counters start at zero; every completed decode leaves them zero).
int scratch_on_current_device(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxScratchDevices) return hip_fail("scratch: device ordinal out of range", hipErrorInvalidDevice);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail("hipGetSymbolAddress(scratch)", e != hipSuccess ? e : hipErrorUnknown);
    const int fe = gqa::launch_fill_words((uint32_t*)p, kScratchBytes / 4, 0u, stream);
    if (fe != 0) return hip_fail("fill_words launch (scratch)", fe);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

gqa::DecodeArgs make_decode_args(const void* q, const void* kc, const void* vc, const int32_t* lens,
                                 int B, int L, int Hq, int Hkv, float scale,
                                 const DecodeShapeCheck& s, void* ws) {
  gqa::DecodeArgs a;
  a.q = (const uint16_t*)q;
  a.kc = (const uint16_t*)kc;
  a.vc = (const uint16_t*)vc;
  a.lens = lens;
  const WsLayout w = ws_layout(B, Hq, s.nsplit);
  a.counters = (int*)ws;
  a.o_part = (float*)((char*)ws + w.o_off);
  a.lse = (float*)((char*)ws + w.lse_off);
  a.out = nullptr;
  a.B = B; a.L = L; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.hgroups = s.hgroups;
  a.chunk = s.chunk;
  a.nsplit = s.nsplit;
  a.c = (float)((double)scale * kLog2e);
  return a;
}

int run_decode(const void* q, const void* kc, const void* vc, const int32_t* lens, void* out,
               int B, int L, int Hq, int Hkv, float scale, const DecodeShapeCheck& s,
               void* ws, hipStream_t stream) {
  gqa::DecodeArgs a = make_decode_args(q, kc, vc, lens, B, L, Hq, Hkv, scale, s, ws);
  a.out = (uint16_t*)out;
  int e = gqa::launch_decode(a, true, stream);
  if (e != 0) return hip_fail("decode launch", e);
  return GQA_ATTN_OK;
}

}  // namespace

extern "C" {

int gqa_attn_version(void) { return GQA_ATTN_VERSION; }

const char* gqa_attn_strerror(int code) {
  switch (code) {
    case GQA_ATTN_OK: return "success";
    case GQA_ATTN_ERR_NULL: return "a required pointer is NULL";
    case GQA_ATTN_ERR_DIM: return "bad dimension or scale (sizes < 1, Hq % Hkv != 0, non-finite scale, or sizes too large)";
    case GQA_ATTN_ERR_UNSUPPORTED: return "unsupported: head dim must be 128 and pointers 16-byte aligned";
    case GQA_ATTN_ERR_HIP: return "HIP launch or allocation failure";
    case GQA_ATTN_ERR_WORKSPACE: return "workspace missing or too small, or split size not a positive multiple of 64";
    default: return "unknown error code";
  }
}

const char* gqa_attn_last_error(void) { return g_last_error.c_str(); }

int gqa_attn_probe_hbm_read(const void* buf, size_t bytes, int workgroups,
                            uint32_t* sink, size_t sink_words, void* stream) {
  if (!buf || !sink) return GQA_ATTN_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > 65535) return GQA_ATTN_ERR_DIM;
  if (!aligned16(buf)) return GQA_ATTN_ERR_UNSUPPORTED;
  if (sink_words < (size_t)workgroups * 256) return GQA_ATTN_ERR_WORKSPACE;
  const int e = gqa::launch_probe_hbm_read(buf, bytes, sink, workgroups, (hipStream_t)stream);
  if (e != 0) return hip_fail("probe_hbm_read launch", e);
  return GQA_ATTN_OK;
}

int gqa_attn_probe_mfma_bf16(int rounds, uint32_t seed, int workgroups,
                             float* sink, size_t sink_floats,
                             uint64_t* ticks, size_t ticks_count, void* stream) {
  if (!sink || !ticks) return GQA_ATTN_ERR_NULL;
  if (rounds < 1 || rounds > (1 << 20) || workgroups < 1 || workgroups > 65535) return GQA_ATTN_ERR_DIM;
  if (sink_floats < (size_t)workgroups * 256 || ticks_count < (size_t)workgroups * 2) return GQA_ATTN_ERR_WORKSPACE;
  const int e = gqa::launch_probe_mfma_bf16(rounds, seed, workgroups, sink, ticks, (hipStream_t)stream);
  if (e != 0) return hip_fail("probe_mfma_bf16 launch", e);
  return GQA_ATTN_OK;
}

// Shape checks and launch plan of a prefill (everything but the pointers).
// form_waves / form_ks: 0 / 0 for the library's choice, else one of the (waves, key
// splits) pairs gqa_attn_prefill_plan reports: (4, 1), (8, 1) or (8, 2).
int plan_prefill(int B, int S, int Hq, int Hkv, int D, float scale, gqa::PrefillArgs* a,
                 int form_waves = 0, int form_ks = 0) {
  if (B < 1 || S < 1) return GQA_ATTN_ERR_DIM;
  int e = check_heads(Hq, Hkv, D, scale);
  if (e) return e;
  if (elems4(B, S, Hq) < 0) return GQA_ATTN_ERR_DIM;
  // The copies of a full K/V tile address row r (r < 64) of the tile with the 32-bit
  // per-lane byte offset r * Hkv * 256 + (chunk slot) * 16; refuse head counts for which
  // that offset would wrap (Hkv >= 266306) instead of reading other rows.
  if ((long long)(gqa::kTileRowsHost - 1) * Hkv * gqa::kRowBytesHost + (gqa::kRowBytesHost - 1) >= (1LL << 32))
    return GQA_ATTN_ERR_DIM;
  a->B = B; a->S = S; a->Hq = Hq; a->Hkv = Hkv; a->G = Hq / Hkv;
  a->nrb = (S + 31) / 32;
  const long long units = (long long)a->G * a->nrb;
  // unit indices (workgroup * waves + wave) are 32-bit in the kernels
  if (units > 0x7fffffffLL - 16) return GQA_ATTN_ERR_DIM;
  if (form_waves == 0 && form_ks == 0) {
    a->nw = gqa::prefill_waves(B, S, Hkv, a->G);
    a->ks = gqa::prefill_key_splits(B, S, Hkv, a->G);
  } else if (form_waves == 4 && form_ks == 1) {
    a->nw = 4; a->ks = 1;
  } else if (form_waves == 8 && form_ks == 1) {
    a->nw = 8; a->ks = 1;
  } else if (form_waves == 8 && form_ks == 2) {
    a->nw = 4; a->ks = 2;        // 4 units per workgroup, two waves each
  } else {
    return GQA_ATTN_ERR_UNSUPPORTED;
  }
  const long long wgs = (units + a->nw - 1) / a->nw;
  const long long grid = wgs * (long long)B * Hkv;
  if (grid > 0x7fffffffLL) return GQA_ATTN_ERR_DIM;
  a->wgs_per_slot = (int)wgs;
  a->nslots = B * Hkv;
  a->c = (float)((double)scale * kLog2e);
  return 0;
}

int gqa_attn_prefill(const void* q, const void* k, const void* v, void* out,
                     int B, int S, int Hq, int Hkv, int D, float scale, int causal,
                     void* stream) {
  return gqa_attn_prefill_form(q, k, v, out, B, S, Hq, Hkv, D, scale, causal, 0, 0, stream);
}

int gqa_attn_prefill_form(const void* q, const void* k, const void* v, void* out,
                          int B, int S, int Hq, int Hkv, int D, float scale, int causal,
                          int waves, int key_splits, void* stream) {
  if (!q || !k || !v || !out) return GQA_ATTN_ERR_NULL;
  gqa::PrefillArgs a;
  int e = plan_prefill(B, S, Hq, Hkv, D, scale, &a, waves, key_splits);
  if (e) return e;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return GQA_ATTN_ERR_UNSUPPORTED;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.out = (uint16_t*)out;
  e = gqa::launch_prefill(a, causal != 0, (hipStream_t)stream);
  if (e != 0) return hip_fail("prefill launch", e);
  return GQA_ATTN_OK;
}

int gqa_attn_prefill_tiles(const void* q, const void* k, const void* v, void* out,
                           int B, int S, int Hq, int Hkv, int D, float scale, int causal,
                           int rows_per_wave, int keys_per_tile, int waves, void* stream) {
  if (!q || !k || !v || !out) return GQA_ATTN_ERR_NULL;
  const int key = 1000 * rows_per_wave + 10 * keys_per_tile + waves;
  const bool product = (key == 32644 || key == 32648);   // the 4- and 8-wave forms
  const bool sweep = (key == 32324 || key == 32328 || key == 33284 || key == 33288 || key == 64324 || key == 64644);
  if (!product && !sweep) return GQA_ATTN_ERR_UNSUPPORTED;
  gqa::PrefillArgs a;
  int e = plan_prefill(B, S, Hq, Hkv, D, scale, &a, product ? waves : 4, 1);
  if (e) return e;
  // 128-key tiles address rows up to 127 with the same 32-bit per-lane offsets
  if ((long long)(keys_per_tile - 1) * Hkv * gqa::kRowBytesHost + (gqa::kRowBytesHost - 1) >= (1LL << 32))
    return GQA_ATTN_ERR_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return GQA_ATTN_ERR_UNSUPPORTED;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.out = (uint16_t*)out;
  if (product) {
    e = gqa::launch_prefill(a, causal != 0, (hipStream_t)stream);
  } else {
    // units (32-row blocks of one head) per workgroup, and the grid for it
    a.nw = waves * rows_per_wave / 32;
    a.ks = 1;
    const long long units = (long long)a.G * a.nrb;
    const long long wgs = (units + a.nw - 1) / a.nw;
    if (wgs * (long long)a.nslots > 0x7fffffffLL) return GQA_ATTN_ERR_DIM;
    a.wgs_per_slot = (int)wgs;
    e = gqa::launch_prefill_tiles(a, causal != 0, rows_per_wave, keys_per_tile, waves, (hipStream_t)stream);
  }
  if (e != 0) return hip_fail("prefill (tile form) launch", e);
  return GQA_ATTN_OK;
}

int gqa_attn_prefill_plan(int B, int S, int Hq, int Hkv, int D, int* waves, int* workgroups,
                          int* key_splits) {
  gqa::PrefillArgs a;
  const int e = plan_prefill(B, S, Hq, Hkv, D, 1.0f, &a);
  if (e) return e;
  if (waves) *waves = a.nw * a.ks;
  if (workgroups) *workgroups = a.wgs_per_slot * a.nslots;
  if (key_splits) *key_splits = a.ks;
  return GQA_ATTN_OK;
}

int gqa_attn_decode_plan(int B, int L, int Hq, int Hkv, int D, int* chunk, int* nsplit) {
  DecodeShapeCheck s = check_decode_shape(B, L, Hq, Hkv, D, 1.0f, 0);
  if (s.code) return s.code;
  if (chunk) *chunk = s.chunk;
  if (nsplit) *nsplit = s.nsplit;
  return GQA_ATTN_OK;
}

size_t gqa_attn_decode_workspace_bytes(int B, int L, int Hq, int Hkv, int D, int chunk) {
  DecodeShapeCheck s = check_decode_shape(B, L, Hq, Hkv, D, 1.0f, chunk);
  if (s.code) return 0;
  return ws_bytes_for(B, Hq, s.nsplit);
}

int gqa_attn_decode(const void* q, const void* kcache, const void* vcache,
                    const int32_t* lens, void* out,
                    int B, int L, int Hq, int Hkv, int D, float scale,
                    void* stream) {
  if (!q || !kcache || !vcache || !lens || !out) return GQA_ATTN_ERR_NULL;
  DecodeShapeCheck s = check_decode_shape(B, L, Hq, Hkv, D, scale, 0);
  if (s.code) return s.code;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(out))
    return GQA_ATTN_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const WsLayout w = ws_layout(B, Hq, s.nsplit);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int e = get_workspace(w.total, (hipStream_t)stream, &ws);
  if (e) return e;
  return run_decode(q, kcache, vcache, lens, out, B, L, Hq, Hkv, scale, s, ws, (hipStream_t)stream);
}

int gqa_attn_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                            const int32_t* lens, void* out,
                            int B, int L, int Hq, int Hkv, int D, float scale,
                            void* stream) {
  if (!q || !kcache || !vcache || !lens || !out) return GQA_ATTN_ERR_NULL;
  DecodeShapeCheck s = check_decode_shape(B, L, Hq, Hkv, D, scale, 0);
  if (s.code) return s.code;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(out))
    return GQA_ATTN_ERR_UNSUPPORTED;
  const size_t need = ws_bytes_for(B, Hq, s.nsplit);
  if (need > kScratchBytes) {
    char buf[160];
    std::snprintf(buf, sizeof(buf), "gqa_attn_decode_noalloc: this shape needs %zu bytes of scratch, more than the %zu "
                  "the library holds per GPU", need, kScratchBytes);
    g_last_error = buf;
    return GQA_ATTN_ERR_WORKSPACE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  void* ws = nullptr;
  const int e = scratch_on_current_device((hipStream_t)stream, &ws);
  if (e) return e;
  return run_decode(q, kcache, vcache, lens, out, B, L, Hq, Hkv, scale, s, ws, (hipStream_t)stream);
}

int gqa_attn_decode_ws(const void* q, const void* kcache, const void* vcache,
                       const int32_t* lens, void* out,
                       int B, int L, int Hq, int Hkv, int D, float scale,
                       int chunk, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !kcache || !vcache || !lens || !out) return GQA_ATTN_ERR_NULL;
  DecodeShapeCheck s = check_decode_shape(B, L, Hq, Hkv, D, scale, chunk);
  if (s.code) return s.code;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(out))
    return GQA_ATTN_ERR_UNSUPPORTED;
  if (!ws || !aligned16(ws) || ws_bytes < ws_bytes_for(B, Hq, s.nsplit)) return GQA_ATTN_ERR_WORKSPACE;
  return run_decode(q, kcache, vcache, lens, out, B, L, Hq, Hkv, scale, s, ws, (hipStream_t)stream);
}

int gqa_attn_decode_partials(const void* q, const void* kcache, const void* vcache,
                             const int32_t* lens, int B, int L, int Hq, int Hkv, int D,
                             float scale, int chunk, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !kcache || !vcache || !lens) return GQA_ATTN_ERR_NULL;
  DecodeShapeCheck s = check_decode_shape(B, L, Hq, Hkv, D, scale, chunk);
  if (s.code) return s.code;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache)) return GQA_ATTN_ERR_UNSUPPORTED;
  if (!ws || !aligned16(ws) || ws_bytes < ws_bytes_for(B, Hq, s.nsplit)) return GQA_ATTN_ERR_WORKSPACE;
  gqa::DecodeArgs a = make_decode_args(q, kcache, vcache, lens, B, L, Hq, Hkv, scale, s, ws);
  int e = gqa::launch_decode(a, false, (hipStream_t)stream);
  if (e != 0) return hip_fail("decode partials launch", e);
  return GQA_ATTN_OK;
}

int gqa_attn_decode_combine(const void* ws, size_t ws_bytes, void* out,
                            int B, int Hq, int D, int nsplit, void* stream) {
  if (!ws || !out) return GQA_ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || nsplit < 1) return GQA_ATTN_ERR_DIM;
  if (nsplit > gqa::kMaxSplits) return GQA_ATTN_ERR_WORKSPACE;
  if (D != 128) return GQA_ATTN_ERR_UNSUPPORTED;
  if (elems4(B, Hq, nsplit) < 0 || B > kMaxGridY || Hq > kMaxGridY) return GQA_ATTN_ERR_DIM;
  if (!aligned16(ws) || !aligned16(out)) return GQA_ATTN_ERR_UNSUPPORTED;
  const WsLayout w = ws_layout(B, Hq, nsplit);
  if (ws_bytes < w.total) return GQA_ATTN_ERR_WORKSPACE;
  gqa::CombineArgs cmb{(const float*)((const char*)ws + w.o_off),
                       (const float*)((const char*)ws + w.lse_off), (uint16_t*)out, B, Hq, nsplit};
  int e = gqa::launch_decode_combine(cmb, (hipStream_t)stream);
  if (e != 0) return hip_fail("decode combine launch", e);
  return GQA_ATTN_OK;
}

void gqa_attn_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if (g_ws.empty() && g_retired.empty()) return;
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (auto& kv : g_ws) {
    if (kv.second.ptr) {
      (void)hipSetDevice(kv.first.first);
      (void)hipFree(kv.second.ptr);
    }
  }
  for (auto& r : g_retired) {
    (void)hipSetDevice(r.first);
    (void)hipFree(r.second);
  }
  g_ws.clear();
  g_retired.clear();
  (void)hipSetDevice(cur);
}

}  // extern "C"
