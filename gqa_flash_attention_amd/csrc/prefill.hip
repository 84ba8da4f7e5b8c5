// prefill.hip - causal / full GQA attention over a prompt on gfx950 (kernel K1).
//
// Implements the prefill mode of the chowfi/kernels README ("Result": process the full
// prompt with a causal mask), with three of the ideas its "What helped most" section
// lists, redone for CDNA4:
//  - item 2 (GQA packing): the waves of a workgroup are the query heads of one KV group
//    (or, for other group sizes, consecutive row blocks), so each K/V tile is staged
//    once into LDS and read by every head that shares it;
//  - item 3 (skip the masked half): a workgroup stops at the last key tile its rows can
//    see, and a wave skips the arithmetic of tiles that lie wholly above its diagonal;
//  - item 4 (largest blocks first): workgroup ids are mapped so the query tiles with the
//    most key tiles start first;
//  - item 5 (exp2 math): the softmax runs in base 2 with scale*log2(e) folded into the
//    logits, on the native v_exp_f32.
//
// Work decomposition. One wave owns 32 query rows of one head and keeps, per lane, one
// query row (lane % 32) and half of the keys of every tile (lane / 32). A workgroup is
// NW = 4 waves (one 32-row block of each head of a KV group; two workgroups per CU) or
// NW = 8 waves (two row blocks; one workgroup per CU). K/V tiles go through a ring of
// 2P stages in LDS, P = NW / 4, and are published P at a time: wait for this wave's
// copies, one barrier, then the copies of the next P tiles into the stages the barrier
// has freed. The 8-wave form copies each tile once for 256 query rows instead of 128
// and meets a barrier every other tile; with a single workgroup per CU a barrier idles
// the whole CU, so halving them is what makes it pay (3-4% at 16K-32K keys on MI355X).
// With one workgroup per CU it needs enough of them to balance the causal triangle: it
// is the faster form from 5/3 workgroups per CU, and shorter prompts keep 4 waves. Where
// even the 4-wave grid holds at most 2 workgroups per CU, the critical path is the
// longest query tile's walk over its keys; there a key-split form (prefill_split_kernel,
// below) gives each set of 4 units a second set of 4 waves that walks the other half of
// the key tiles.
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K from LDS
// is the A operand, the wave's Q rows stay in registers as the B operand. In that layout each
// lane's 32 scores of a 64-key tile belong to its own query row, so the row max needs
// only one exchange between the two wave halves. The probabilities are rounded to bf16
// in place and fed, with no data movement, as the B operand of O^T += V^T P^T; V^T comes
// from LDS through ds_read_b64_tr_b16.
//
// Online softmax (per query row, fp32): running max m (log2 units), partial sum l, and
// the accumulator O. The rescale of O is lazy: m only moves when a tile raises the row
// max by more than kTau, so most tiles skip the 64 multiplies; numerator and denominator
// always share the same m, so the result is unchanged.
#include "gqa_device.hpp"
#include "gqa_internal.hpp"

namespace gqa {

constexpr float kTau = 8.0f;   // lazy-rescale threshold, log2 units (p <= 2^8)

// Online-softmax state of one wave's 32 query rows: running max m (log2 units), this
// lane's partial sum l over its half of the keys, and O^T (lane: one query row, 64 of its
// 128 output columns), all relative to m.
struct RowState {
  float m;
  float l;
  f32x16 o[4];
};

struct NoHook {
  __device__ void operator()() const {}
};

// One 64-key tile of K (kt) and V (vt) in LDS, key tile index t, for the wave whose 32
// query rows start at q0 and whose Q fragments are qreg (B operand, 8 k-steps of 16 d).
// after_qk() runs once the tile's Q.K^T MFMAs have issued.
template <bool CAUSAL, bool POS, typename Hook = NoHook>
__device__ __forceinline__ void attend_tile(const GQA_LDS uint8_t* kt, const GQA_LDS uint8_t* vt,
                                            int t, int q0, int S, float c, int lane,
                                            const bf16x8 (&qreg)[8], RowState& st,
                                            Hook after_qk = Hook{}) {
  const int h = lane >> 5;
  const int qi = lane & 31;
  // S^T[key][query] for the tile's 64 keys, two 32-key blocks. The K operand reads run
  // 4 k-steps ahead of the MFMAs that consume them. The wave raises its issue priority
  // while it feeds the matrix cores, so that on a SIMD shared with a wave doing softmax
  // work the MFMA stream is not starved.
  __builtin_amdgcn_s_setprio(1);
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  bf16x8 ka[4], kb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    ka[ks] = lds_read_k(kt, qi, 2 * ks + h);
    kb[ks] = lds_read_k(kt, 32 + qi, 2 * ks + h);
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    s0 = mfma32(ka[ks & 3], qreg[ks], s0);
    s1 = mfma32(kb[ks & 3], qreg[ks], s1);
    if (ks + 4 < 8) {
      ka[ks & 3] = lds_read_k(kt, qi, 2 * (ks + 4) + h);
      kb[ks & 3] = lds_read_k(kt, 32 + qi, 2 * (ks + 4) + h);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  after_qk();
  if (!POS) {
#pragma unroll
    for (int v = 0; v < 16; ++v) { s0[v] *= c; s1[v] *= c; }
  }
  // Mask keys this lane's query may not see: above the diagonal (causal) or past S.
  const int key0 = t * kTileRows;
  const bool need_mask = CAUSAL ? (key0 + kTileRows - 1 > q0) : (key0 + kTileRows > S);
  if (need_mask) {
    const int lim = CAUSAL ? (q0 + qi) : (S - 1);   // largest visible key
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kk = key0 + 8 * (v >> 2) + 4 * h + (v & 3);
      if (kk > lim) s0[v] = -INFINITY;
      if (kk + 32 > lim) s1[v] = -INFINITY;
    }
  }
  float mx = s0[0];
#pragma unroll
  for (int v = 1; v < 16; ++v) mx = vmax(mx, s0[v]);
#pragma unroll
  for (int v = 0; v < 16; ++v) mx = vmax(mx, s1[v]);
  mx = halves_max(mx);
  const float m_cand = vmax(st.m, POS ? mx * c : mx);
  const bool upd = m_cand > st.m + kTau;
  if (__builtin_amdgcn_ballot_w64(upd) != 0) {
    const float m_new = upd ? m_cand : st.m;
    const float alpha = (m_new == st.m) ? 1.f : exp2_fast(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) st.o[mb] *= alpha;
    st.m = m_new;
  }
  const float neg_m = -st.m;
  // O^T[d][query] += V^T[d][key] P^T[key][query], 4 k-steps of 16 keys. P^T is the B
  // operand straight from the accumulator layout (k index 8h+u <-> key
  // 16t4 + 8(u/4) + 4h + u%4). For d-block mb the A operand has lane l holding
  // d = 32mb + l%32 and keys 16t4 + 4(l/32) + {0..3, 8..11}, read transposed from LDS.
  // Each step's probabilities are formed just before its MFMAs and the next step's V
  // reads are already in flight, so exp work overlaps the matrix cores.
  const int g16 = lane >> 4;
  const int li = lane & 15;
  const int vrow = 4 * (g16 >> 1) + (li >> 2);
  const int vcol = 16 * (g16 & 1) + 4 * (li & 3);
  s16x4 vlo[4], vhi[4];
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    vlo[mb] = lds_read_v_tr(vt, vrow, 32 * mb + vcol);
    vhi[mb] = lds_read_v_tr(vt, 8 + vrow, 32 * mb + vcol);
  }
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) {
    const f32x16& sb = (t4 < 2) ? s0 : s1;
    const int o = 8 * (t4 & 1);
    float e[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      e[u] = exp2_fast(POS ? __builtin_fmaf(sb[o + u], c, neg_m) : sb[o + u] + neg_m);
    const bf16x8 p = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    st.l = sum_bf16x8(p, st.l);
    s16x4 nlo[4], nhi[4];
    if (t4 < 3) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        nlo[mb] = lds_read_v_tr(vt, 16 * (t4 + 1) + vrow, 32 * mb + vcol);
        nhi[mb] = lds_read_v_tr(vt, 16 * (t4 + 1) + 8 + vrow, 32 * mb + vcol);
      }
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) st.o[mb] = mfma32(join_bf16x8(vlo[mb], vhi[mb]), p, st.o[mb]);
    if (t4 < 3) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) { vlo[mb] = nlo[mb]; vhi[mb] = nhi[mb]; }
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

// Row qpos of head `head`: this lane's 64 output columns of O / l as bf16.
__device__ __forceinline__ void store_rows(const PrefillArgs& a, int b, int qpos, int head, int h,
                                           float l_tot, const RowState& st) {
  const float inv = 1.0f / l_tot;
  uint16_t* op = a.out + (((size_t)b * a.S + qpos) * a.Hq + head) * kD + 4 * h;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) {
      typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
      u16x4 w;
      w[0] = bf16_bits(st.o[mb][4 * vq + 0] * inv);
      w[1] = bf16_bits(st.o[mb][4 * vq + 1] * inv);
      w[2] = bf16_bits(st.o[mb][4 * vq + 2] * inv);
      w[3] = bf16_bits(st.o[mb][4 * vq + 3] * inv);
      *(u16x4*)(op + 32 * mb + 8 * vq) = w;
    }
  }
}

template <bool CAUSAL, bool POS, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a) {
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  constexpr int P = NW / 4;      // tiles published per barrier
  constexpr int NST = 2 * P;     // ring stages, one K tile and one V tile each
  __shared__ __attribute__((aligned(1024))) uint8_t lds_kv[NST][2][kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;      // which half of every 64-key tile this lane holds
  const int qi = lane & 31;     // this lane's query row within the wave's 32 rows

  // Workgroup -> (batch, KV head, query tile). Consecutive ids go to different (b, g)
  // slots; with 8 KV heads and round-robin dispatch over 8 XCDs each XCD then serves one
  // KV head, whose K/V stays in that XCD's L2. Within a slot, ids run over query tiles
  // from the last (most key tiles) to the first.
  const int bid = blockIdx.x;
  const int slot = bid % a.nslots;
  const int j = bid / a.nslots;
  const int wg = CAUSAL ? (a.wgs_per_slot - 1 - j) : j;
  const int b = slot / a.Hkv;
  const int g = slot % a.Hkv;
  const int nunits = a.G * a.nrb;
  const int unit = NW * wg + wave;
  const bool active = unit < nunits;
  const int rb = active ? unit / a.G : 0;
  const int head = g * a.G + (active ? unit % a.G : 0);
  const int q0 = rb * 32;

  const int last_unit = min(NW * wg + NW - 1, nunits - 1);
  const int kv_end = CAUSAL ? min(a.S, (last_unit / a.G) * 32 + 32) : a.S;
  const int nt = (kv_end + kTileRows - 1) / kTileRows;
  const int own_end = CAUSAL ? min(a.S, q0 + 32) : a.S;
  const int own_nt = (own_end + kTileRows - 1) / kTileRows;

  const size_t kv_stride = (size_t)a.Hkv * kD;
  const uint16_t* kbase = a.k + ((size_t)b * a.S * a.Hkv + g) * kD;
  const uint16_t* vbase = a.v + ((size_t)b * a.S * a.Hkv + g) * kD;

  TileCopy<NW> copy;
  copy.init(kv_stride, wave, lane);
  // Copies of tile t (K then V): the per-lane offsets for a full tile, the clamped
  // per-row path for the ragged last tile.
  auto issue_tile = [&](int t, GQA_LDS uint8_t* kd, GQA_LDS uint8_t* vd) {
    const int r0 = t * kTileRows;
    if (kv_end - r0 >= kTileRows) {
      copy.issue_full(kd, vd, kbase + (size_t)r0 * kv_stride, vbase + (size_t)r0 * kv_stride, wave);
    } else {
      stage_tile<NW, false>(kd, kbase + (size_t)r0 * kv_stride, kv_stride, kv_end - r0, wave, lane);
      stage_tile<NW, true>(vd, vbase + (size_t)r0 * kv_stride, kv_stride, kv_end - r0, wave, lane);
    }
  };

  auto kbuf = [&](int st) { return (GQA_LDS uint8_t*)lds_kv[st][0]; };
  auto vbuf = [&](int st) { return (GQA_LDS uint8_t*)lds_kv[st][1]; };
  // Prologue: start tile 0, then fetch this wave's Q rows (B operand, 8 k-steps of 16 d).
  issue_tile(0, kbuf(0), vbuf(0));
  bf16x8 qreg[8];
  {
    const int qrow = min(q0 + qi, a.S - 1);
    const uint16_t* qp = a.q + (((size_t)b * a.S + qrow) * a.Hq + head) * kD + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = *(const bf16x8*)(qp + 16 * ks);
  }
  // Q and tile 0 have landed. Waiting here also tells the compiler that no load of its
  // own is outstanding inside the loop, so it adds no waits there. Then tiles 1..P-1.
  wait_vmcnt<0>();
#pragma unroll
  for (int t = 1; t < P; ++t)
    if (t < nt) issue_tile(t, kbuf(t), vbuf(t));

  RowState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) st.o[mb] = f32x16{};

  // One key tile. BUF = t % NST selects the ring stage at compile time.
  auto step = [&](int t, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    GQA_LDS uint8_t* const kt = kbuf(BUF);
    GQA_LDS uint8_t* const vt = vbuf(BUF);
    // At t = 0 mod P this wave's copies of tiles t .. t+P-1 (the only ones in flight)
    // land; after the barrier every wave's have, and every wave is done with tiles
    // t-P .. t-1: their LDS reads fed MFMAs that have issued, so they have completed.
    // Their stages then take tiles t+P .. t+2P-1.
    auto issue_next = [&]() {
      if (BUF % P == 0) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const int nx = (BUF + P + i) % NST;
          if (t + P + i < nt) issue_tile(t + P + i, kbuf(nx), vbuf(nx));
        }
      }
    };
    if (BUF % P == 0) {
      wait_vmcnt<0>();
      tile_barrier();
    }
    // The 4-wave form needs the next tile at the next step, so its copies go out at once.
    // The 8-wave form has two steps of slack and issues them after this tile's Q.K^T
    // MFMAs, so the copies' LDS writes do not compete with the K reads that start the
    // step (1% faster at 8K-32K keys on MI355X).
    if (P == 1) issue_next();
    if (!active || t >= own_nt) {
      if (P > 1) issue_next();
      return;
    }
    if (P > 1) attend_tile<CAUSAL, POS>(kt, vt, t, q0, a.S, a.c, lane, qreg, st, issue_next);
    else       attend_tile<CAUSAL, POS>(kt, vt, t, q0, a.S, a.c, lane, qreg, st);
  };

  for (int t = 0; t < nt; t += NST) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nt) step(t + 1, std::integral_constant<int, 1 % NST>{});
    if (NST > 2 && t + 2 < nt) step(t + 2, std::integral_constant<int, 2 % NST>{});
    if (NST > 3 && t + 3 < nt) step(t + 3, std::integral_constant<int, 3 % NST>{});
  }

  // Epilogue: the two halves of the wave hold disjoint keys of the same rows.
  const float l_tot = halves_sum(st.l);
  if (!active) return;
  const int qpos = q0 + qi;
  if (qpos >= a.S) return;
  store_rows(a, b, qpos, head, h, l_tot, st);
}

// Key-split form, for grids too small to fill the GPU (short prompts). A workgroup of 8
// waves serves the same 4 (row block, head) units as the 4-wave form, but its two halves
// of 4 waves take different halves of the units' key tiles, the first ceil(nt/2) and the
// rest, one tile per step through a 2-stage ring of their own. Each half keeps its own
// online softmax; at the end half 1 hands (m, l, O) to half 0 through LDS, and half 0
// merges the two by their log-sum-exp weights and writes the rows. The longest job of the
// causal triangle then takes half the steps, and every SIMD holds two waves.
template <bool CAUSAL, bool POS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_split_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_kv[2][2][2][kTileBytes];   // [half][stage][K/V]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave >> 2;   // which half of the key tiles this wave streams
  const int sub = wave & 3;     // the wave's unit within the workgroup
  const int h = lane >> 5;
  const int qi = lane & 31;

  // Workgroup -> (batch, KV head, query tile) exactly as in the 4-wave form.
  const int bid = blockIdx.x;
  const int slot = bid % a.nslots;
  const int j = bid / a.nslots;
  const int wg = CAUSAL ? (a.wgs_per_slot - 1 - j) : j;
  const int b = slot / a.Hkv;
  const int g = slot % a.Hkv;
  const int nunits = a.G * a.nrb;
  const int unit = 4 * wg + sub;
  const bool active = unit < nunits;
  const int rb = active ? unit / a.G : 0;
  const int head = g * a.G + (active ? unit % a.G : 0);
  const int q0 = rb * 32;

  const int last_unit = min(4 * wg + 3, nunits - 1);
  const int kv_end = CAUSAL ? min(a.S, (last_unit / a.G) * 32 + 32) : a.S;
  const int nt = (kv_end + kTileRows - 1) / kTileRows;
  const int mid = (nt + 1) / 2;               // half 0: tiles [0, mid); half 1: [mid, nt)
  const int t_begin = half ? mid : 0;
  const int t_end = half ? nt : mid;
  const int own_end = CAUSAL ? min(a.S, q0 + 32) : a.S;
  const int own_nt = (own_end + kTileRows - 1) / kTileRows;

  const size_t kv_stride = (size_t)a.Hkv * kD;
  const uint16_t* kbase = a.k + ((size_t)b * a.S * a.Hkv + g) * kD;
  const uint16_t* vbase = a.v + ((size_t)b * a.S * a.Hkv + g) * kD;

  TileCopy<4> copy;
  copy.init(kv_stride, sub, lane);
  auto kbuf = [&](int stage) { return (GQA_LDS uint8_t*)lds_kv[half][stage][0]; };
  auto vbuf = [&](int stage) { return (GQA_LDS uint8_t*)lds_kv[half][stage][1]; };
  // Copies of tile t by this half's 4 waves.
  auto issue_tile = [&](int t, GQA_LDS uint8_t* kd, GQA_LDS uint8_t* vd) {
    const int r0 = t * kTileRows;
    if (kv_end - r0 >= kTileRows) {
      copy.issue_full(kd, vd, kbase + (size_t)r0 * kv_stride, vbase + (size_t)r0 * kv_stride, sub);
    } else {
      stage_tile<4, false>(kd, kbase + (size_t)r0 * kv_stride, kv_stride, kv_end - r0, sub, lane);
      stage_tile<4, true>(vd, vbase + (size_t)r0 * kv_stride, kv_stride, kv_end - r0, sub, lane);
    }
  };

  if (t_begin < t_end) issue_tile(t_begin, kbuf(0), vbuf(0));
  bf16x8 qreg[8];
  {
    const int qrow = min(q0 + qi, a.S - 1);
    const uint16_t* qp = a.q + (((size_t)b * a.S + qrow) * a.Hq + head) * kD + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = *(const bf16x8*)(qp + 16 * ks);
  }
  wait_vmcnt<0>();

  RowState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) st.o[mb] = f32x16{};

  // Step i: this half's tile t = t_begin + i. Both halves take the same barrier each step
  // (half 1 has at most as many tiles as half 0); their rings are disjoint. The barrier
  // publishes tile t and frees the stage tile t - 1 used, which takes tile t + 1.
  auto step = [&](int i, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int t = t_begin + i;
    wait_vmcnt<0>();
    tile_barrier();
    if (t + 1 < t_end) issue_tile(t + 1, kbuf(BUF ^ 1), vbuf(BUF ^ 1));
    if (!active || t >= t_end || t >= own_nt) return;
    attend_tile<CAUSAL, POS>(kbuf(BUF), vbuf(BUF), t, q0, a.S, a.c, lane, qreg, st);
  };
  for (int i = 0; i < mid; i += 2) {
    step(i, std::integral_constant<int, 0>{});
    if (i + 1 < mid) step(i + 1, std::integral_constant<int, 1>{});
  }

  // Merge. Every copy has landed (each was waited for before the barrier of its step) and
  // no wave reads the rings any more, so they hold half 1's state: per lane its 64 O
  // values, m and l, at a stride of 66 floats.
  __syncthreads();
  float* const xs = (float*)lds_kv + ((size_t)sub * 64 + lane) * 66;
  if (half == 1) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) xs[16 * mb + v] = st.o[mb][v];
    xs[64] = st.m;
    xs[65] = st.l;
  }
  __syncthreads();
  if (half == 1 || !active) return;
  {
    // Both parts are relative to their own m; an empty part (m = -inf) weighs nothing.
    const float m1 = xs[64];
    const float mm = fmaxf(st.m, m1);
    const float w0 = (st.m == -INFINITY) ? 0.f : exp2_fast(st.m - mm);
    const float w1 = (m1 == -INFINITY) ? 0.f : exp2_fast(m1 - mm);
    st.l = w0 * st.l + w1 * xs[65];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) st.o[mb][v] = w0 * st.o[mb][v] + w1 * xs[16 * mb + v];
  }
  const float l_tot = halves_sum(st.l);
  const int qpos = q0 + qi;
  if (qpos >= a.S) return;
  store_rows(a, b, qpos, head, h, l_tot, st);
}

// ----------------------------------------------------------------------------------------
// Other tile shapes, for the tile-shape sweep (gqa_attn_prefill_tiles). The forms above use
// 64-key tiles and 32 query rows per wave; here the key tile holds BN = 32 * NB keys
// (NB = 1, 2 or 4 blocks of 32) and a wave owns NQ = 1 or 2 units of 32 rows (BM = 32 * NQ
// rows per wave), with every K and V fragment read from LDS feeding the MFMAs of all NQ
// units. The arithmetic per unit is the product's: S^T = K Q^T, base-2 online softmax with
// the lazy rescale, bf16 P into O^T += V^T P^T. With NQ = 2 a wave carries twice the state
// (about 300 registers) and runs alone on its SIMD.
// ----------------------------------------------------------------------------------------

// Copies of a full BN-row K/V tile, per-lane offsets computed once (as TileCopy does for
// 64 rows): instruction j of wave w fills rows 4 (w + NW j) .. +3.
template <int NW, int BN>
struct TileCopyN {
  static constexpr int kPer = (BN / 4) / NW;
  static_assert(kPer >= 1 && (BN / 4) % NW == 0, "tile rows per wave");
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
  __device__ __forceinline__ void issue_full(GQA_LDS uint8_t* kt, GQA_LDS uint8_t* vt, const uint16_t* kg,
                                             const uint16_t* vg, int wave) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) lds_dma16_sv(kg, ko[j], kt + (wave + NW * j) * 1024);
#pragma unroll
    for (int j = 0; j < kPer; ++j) lds_dma16_sv(vg, vo[j], vt + (wave + NW * j) * 1024);
  }
};

// A ragged BN-row tile: rows at or past nvalid read row nvalid - 1 (nvalid >= 1).
template <int NW, int BN, bool VTILE>
__device__ __forceinline__ void stage_tile_n(GQA_LDS uint8_t* tile, const uint16_t* rows, size_t row_stride,
                                             int nvalid, int wave, int lane) {
#pragma unroll
  for (int i = wave; i < BN / 4; i += NW) {
    const int r = 4 * i + (lane >> 4);
    const int slot = lane & 15;
    const int c = slot ^ (VTILE ? swz_v(r) : swz_k(r));
    const int gr = r < nvalid ? r : nvalid - 1;
    lds_dma16(rows + (size_t)gr * row_stride + c * 8, tile + i * 1024);
  }
}

// One BN-key tile for the NQ units of a wave (query rows q0[u] .. q0[u] + 31 of their
// heads, Q fragments qreg[u]).
template <bool CAUSAL, bool POS, int NB, int NQ>
__device__ __forceinline__ void attend_tile_n(const GQA_LDS uint8_t* kt, const GQA_LDS uint8_t* vt, int t,
                                              const int (&q0)[NQ], int S, float c, int lane,
                                              const bf16x8 (&qreg)[NQ][8], RowState (&st)[NQ]) {
  constexpr int BN = 32 * NB;
  const int h = lane >> 5;
  const int qi = lane & 31;
  __builtin_amdgcn_s_setprio(1);
  f32x16 s[NQ][NB];
#pragma unroll
  for (int u = 0; u < NQ; ++u)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[u][nb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 kf = lds_read_k(kt, 32 * nb + qi, 2 * ks + h);
#pragma unroll
      for (int u = 0; u < NQ; ++u) s[u][nb] = mfma32(kf, qreg[u][ks], s[u][nb]);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  const int key0 = t * BN;
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    if (!POS) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[u][nb][v] *= c;
    }
    const bool need_mask = CAUSAL ? (key0 + BN - 1 > q0[u]) : (key0 + BN > S);
    if (need_mask) {
      const int lim = CAUSAL ? (q0[u] + qi) : (S - 1);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (key0 + 32 * nb + 8 * (v >> 2) + 4 * h + (v & 3) > lim) s[u][nb][v] = -INFINITY;
    }
    float mx = s[u][0][0];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = vmax(mx, s[u][nb][v]);
    mx = halves_max(mx);
    const float m_cand = vmax(st[u].m, POS ? mx * c : mx);
    const bool upd = m_cand > st[u].m + kTau;
    if (__builtin_amdgcn_ballot_w64(upd) != 0) {
      const float m_new = upd ? m_cand : st[u].m;
      const float alpha = (m_new == st[u].m) ? 1.f : exp2_fast(st[u].m - m_new);
      st[u].l *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) st[u].o[mb] *= alpha;
      st[u].m = m_new;
    }
  }
  const int g16 = lane >> 4;
  const int li = lane & 15;
  const int vrow = 4 * (g16 >> 1) + (li >> 2);
  const int vcol = 16 * (g16 & 1) + 4 * (li & 3);
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int t4 = 0; t4 < 2 * NB; ++t4) {
    s16x4 vlo[4], vhi[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      vlo[mb] = lds_read_v_tr(vt, 16 * t4 + vrow, 32 * mb + vcol);
      vhi[mb] = lds_read_v_tr(vt, 16 * t4 + 8 + vrow, 32 * mb + vcol);
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const f32x16& sb = s[u][t4 >> 1];
      const int o = 8 * (t4 & 1);
      const float neg_m = -st[u].m;
      float e[8];
#pragma unroll
      for (int w = 0; w < 8; ++w)
        e[w] = exp2_fast(POS ? __builtin_fmaf(sb[o + w], c, neg_m) : sb[o + w] + neg_m);
      const bf16x8 p = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      st[u].l = sum_bf16x8(p, st[u].l);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) st[u].o[mb] = mfma32(join_bf16x8(vlo[mb], vhi[mb]), p, st[u].o[mb]);
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

// The prefill with BN-key tiles and NQ units (32 rows each) per wave, NW waves per
// workgroup, all units of one KV head (workgroup ids as in prefill_kernel, longest first).
// Each barrier publishes max(1, KB / BN) tiles, KB = 64 * (NW / 4) * NQ keys, through a
// ring of twice that many stages (64 KB of LDS for NW = 4, NQ = 1, BN <= 64; 128 KB else).
template <bool CAUSAL, bool POS, int NW, int NB, int NQ>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NQ == 1 && NW == 8 ? 2 : 1, 2)))
void prefill_tiles_kernel(PrefillArgs a) {
  constexpr int BN = 32 * NB;
  constexpr int KB = 64 * (NW / 4) * NQ;
  constexpr int P = KB / BN >= 1 ? KB / BN : 1;
  constexpr int NST = 2 * P;
  constexpr int kStage = BN * kRowBytes;   // bytes of one K (or V) tile
  __shared__ __attribute__((aligned(1024))) uint8_t lds_kv[NST][2][kStage];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int qi = lane & 31;
  const int bid = blockIdx.x;
  const int slot = bid % a.nslots;
  const int j = bid / a.nslots;
  const int wg = CAUSAL ? (a.wgs_per_slot - 1 - j) : j;
  const int b = slot / a.Hkv;
  const int g = slot % a.Hkv;
  const int nunits = a.G * a.nrb;
  int unit[NQ], q0[NQ], head[NQ];
  bool live[NQ];
  int own_nt = 0;
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    unit[u] = NQ * (NW * wg + wave) + u;
    live[u] = unit[u] < nunits;
    const int rb = live[u] ? unit[u] / a.G : 0;
    head[u] = g * a.G + (live[u] ? unit[u] % a.G : 0);
    q0[u] = rb * 32;
    if (live[u]) own_nt = max(own_nt, ((CAUSAL ? min(a.S, q0[u] + 32) : a.S) + BN - 1) / BN);
  }
  const int last_unit = min(NQ * NW * wg + NQ * NW - 1, nunits - 1);
  const int kv_end = CAUSAL ? min(a.S, (last_unit / a.G) * 32 + 32) : a.S;
  const int nt = (kv_end + BN - 1) / BN;

  const size_t kv_stride = (size_t)a.Hkv * kD;
  const uint16_t* kbase = a.k + ((size_t)b * a.S * a.Hkv + g) * kD;
  const uint16_t* vbase = a.v + ((size_t)b * a.S * a.Hkv + g) * kD;
  TileCopyN<NW, BN> copy;
  copy.init(kv_stride, wave, lane);
  auto kbuf = [&](int st) { return (GQA_LDS uint8_t*)lds_kv[st][0]; };
  auto vbuf = [&](int st) { return (GQA_LDS uint8_t*)lds_kv[st][1]; };
  auto issue_tile = [&](int t, int st) {
    const int r0 = t * BN;
    if (kv_end - r0 >= BN) {
      copy.issue_full(kbuf(st), vbuf(st), kbase + (size_t)r0 * kv_stride, vbase + (size_t)r0 * kv_stride, wave);
    } else {
      stage_tile_n<NW, BN, false>(kbuf(st), kbase + (size_t)r0 * kv_stride, kv_stride, kv_end - r0, wave, lane);
      stage_tile_n<NW, BN, true>(vbuf(st), vbase + (size_t)r0 * kv_stride, kv_stride, kv_end - r0, wave, lane);
    }
  };

  issue_tile(0, 0);
  bf16x8 qreg[NQ][8];
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int qrow = min(q0[u] + qi, a.S - 1);
    const uint16_t* qp = a.q + (((size_t)b * a.S + qrow) * a.Hq + head[u]) * kD + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[u][ks] = *(const bf16x8*)(qp + 16 * ks);
  }
  wait_vmcnt<0>();
  for (int t = 1; t < P; ++t)
    if (t < nt) issue_tile(t, t);

  RowState st[NQ];
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    st[u].m = -INFINITY;
    st[u].l = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) st[u].o[mb] = f32x16{};
  }
  for (int t = 0; t < nt; ++t) {
    const int buf = t % NST;
    if (buf % P == 0) {
      // this wave's copies of tiles t .. t+P-1 land; after the barrier every wave's have,
      // and every wave is done with the stages of tiles t-P .. t-1, which take t+P .. t+2P-1
      wait_vmcnt<0>();
      tile_barrier();
      for (int i = 0; i < P; ++i)
        if (t + P + i < nt) issue_tile(t + P + i, (buf + P + i) % NST);
    }
    if (t < own_nt) attend_tile_n<CAUSAL, POS, NB, NQ>(kbuf(buf), vbuf(buf), t, q0, a.S, a.c, lane, qreg, st);
  }
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const float l_tot = halves_sum(st[u].l);
    const int qpos = q0[u] + qi;
    if (live[u] && qpos < a.S) store_rows(a, b, qpos, head[u], h, l_tot, st[u]);
  }
}

template <int NW, int NB, int NQ>
static void launch_prefill_tiles_form(const PrefillArgs& a, bool causal, hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)a.nslots * a.wgs_per_slot));
  const dim3 block(64 * NW);
  const bool pos = a.c > 0.f;
  if (causal) {
    if (pos) hipLaunchKernelGGL((prefill_tiles_kernel<true, true, NW, NB, NQ>), grid, block, 0, stream, a);
    else     hipLaunchKernelGGL((prefill_tiles_kernel<true, false, NW, NB, NQ>), grid, block, 0, stream, a);
  } else {
    if (pos) hipLaunchKernelGGL((prefill_tiles_kernel<false, true, NW, NB, NQ>), grid, block, 0, stream, a);
    else     hipLaunchKernelGGL((prefill_tiles_kernel<false, false, NW, NB, NQ>), grid, block, 0, stream, a);
  }
}

int launch_prefill_tiles(const PrefillArgs& a, bool causal, int rows_per_wave, int keys_per_tile, int waves,
                         hipStream_t stream) {
  const int key = 1000 * rows_per_wave + 10 * keys_per_tile + waves;
  switch (key) {
    case 32324: launch_prefill_tiles_form<4, 1, 1>(a, causal, stream); break;
    case 32328: launch_prefill_tiles_form<8, 1, 1>(a, causal, stream); break;
    case 33284: launch_prefill_tiles_form<4, 4, 1>(a, causal, stream); break;
    case 33288: launch_prefill_tiles_form<8, 4, 1>(a, causal, stream); break;
    case 64324: launch_prefill_tiles_form<4, 1, 2>(a, causal, stream); break;
    case 64644: launch_prefill_tiles_form<4, 2, 2>(a, causal, stream); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int prefill_waves(int B, int S, int Hkv, int G) {
  // 8 waves once their grid holds at least 5/3 workgroups per CU (B = 1, 32 query and 8
  // KV heads: S > 3392). Paired timing on MI355X against the 4-wave form: x0.97 at 3072
  // keys, x0.99 at 3328, x1.00 at 3456, x1.03 at 4096 and x1.04 at 8128.
  const long long units = (long long)G * ((S + 31) / 32);
  const long long wgs8 = (long long)B * Hkv * ((units + 7) / 8);
  return 3 * wgs8 >= 5 * 256 ? 8 : 4;
}

int prefill_key_splits(int B, int S, int Hkv, int G) {
  // Split the key tiles over two half-workgroups when the 4-wave grid holds at most 2
  // workgroups per CU and the longest job has at least 8 key tiles (B = 1, 32 query and
  // 8 KV heads: 512 <= S <= 2048). On MI355X that is 5-21% faster there; at 3000-4096
  // keys, with 3-4 workgroups per CU, the 4-wave form is 7-8% faster.
  const long long units = (long long)G * ((S + 31) / 32);
  const long long wgs4 = (long long)B * Hkv * ((units + 3) / 4);
  return (prefill_waves(B, S, Hkv, G) == 4 && wgs4 <= 2 * 256 && S >= 512) ? 2 : 1;
}

template <int NW>
static void launch_prefill_nw(const PrefillArgs& a, bool causal, hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)a.nslots * a.wgs_per_slot));
  const dim3 block(64 * NW);
  const bool pos = a.c > 0.f;
  if (causal) {
    if (pos) hipLaunchKernelGGL((prefill_kernel<true, true, NW>), grid, block, 0, stream, a);
    else     hipLaunchKernelGGL((prefill_kernel<true, false, NW>), grid, block, 0, stream, a);
  } else {
    if (pos) hipLaunchKernelGGL((prefill_kernel<false, true, NW>), grid, block, 0, stream, a);
    else     hipLaunchKernelGGL((prefill_kernel<false, false, NW>), grid, block, 0, stream, a);
  }
}

static void launch_prefill_split(const PrefillArgs& a, bool causal, hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)a.nslots * a.wgs_per_slot));
  const dim3 block(512);
  const bool pos = a.c > 0.f;
  if (causal) {
    if (pos) hipLaunchKernelGGL((prefill_split_kernel<true, true>), grid, block, 0, stream, a);
    else     hipLaunchKernelGGL((prefill_split_kernel<true, false>), grid, block, 0, stream, a);
  } else {
    if (pos) hipLaunchKernelGGL((prefill_split_kernel<false, true>), grid, block, 0, stream, a);
    else     hipLaunchKernelGGL((prefill_split_kernel<false, false>), grid, block, 0, stream, a);
  }
}

int launch_prefill(const PrefillArgs& a, bool causal, hipStream_t stream) {
  if (a.nw == 8)      launch_prefill_nw<8>(a, causal, stream);
  else if (a.ks == 2) launch_prefill_split(a, causal, stream);
  else                launch_prefill_nw<4>(a, causal, stream);
  return (int)hipGetLastError();
}

}  // namespace gqa
