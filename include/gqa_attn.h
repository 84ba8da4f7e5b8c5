/*
 * gqa_attn.h - C ABI of the MI355X (gfx950) grouped-query attention forward library.
 *
 * The library computes the forward pass of grouped-query attention (GQA) in its
 * two modes: causal prefill over a full prompt and single-token decode against a
 * KV cache (chowfi/kernels README, "Result": the two mode bullets and the
 * settings line, bf16 with 32 query heads sharing 8 KV heads of size 128).
 *
 * Definition (the page names the operation but writes no formula; it is
 * benchmarked as the same function as FlashAttention-2 and PyTorch SDPA, so the
 * standard one is taken). For batch b, query head h and KV head g(h) = h / (Hq/Hkv):
 *     x[i,j]    = scale * dot(Q[b,i,h,:], K[b,j,g(h),:])       for visible j
 *     out[i,:]  = sum_j softmax_j(x[i,:]) * V[b,j,g(h),:]
 * Prefill, causal: query i sees keys 0..i. Prefill, non-causal: keys 0..S-1.
 * Decode: the one query of sequence b sees cache slots 0..lens[b]-1.
 *
 * Conventions shared by every entry point:
 *  - Tensors are contiguous, device-resident and 16-byte aligned. bf16 values
 *    are passed as raw uint16 bit patterns. The caller owns every tensor.
 *  - Only D = 128 is supported. Hq must be a multiple of Hkv.
 *  - Arithmetic: bf16 operands into matrix cores with fp32 accumulation; the
 *    softmax max, sum and the output accumulator are fp32; outputs are rounded
 *    to bf16 (round to nearest even).
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    on that stream only and calls return without a host synchronisation. A
 *    fault inside a kernel surfaces at the caller's next synchronisation.
 *  - Arguments are validated before any HIP call, so every error code below
 *    except GQA_ATTN_ERR_HIP can be produced on a machine without a GPU.
 *  - Results are bitwise deterministic for a fixed shape, scale and split
 *    count: no reduction uses atomics (the decode's atomic only elects the
 *    workgroup that merges; the merge order is fixed).
 *  - Entry points may be called from several host threads. Calls that share
 *    a stream are ordered by that stream.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define GQA_ATTN_OK               0
#define GQA_ATTN_ERR_NULL        -1  /* a required pointer is NULL                                  */
#define GQA_ATTN_ERR_DIM         -2  /* B, S, L, Hq or Hkv < 1; Hq % Hkv != 0; non-finite scale;
                                        a size whose element count overflows 64-bit offsets; a
                                        launch grid past the device limits (more than 2^31-1
                                        workgroups, or B or Hkv x ceil(G/16) above 65535 for a
                                        decode); a prefill with Hkv >= 266306 (the byte offset
                                        63 x Hkv x 256 of a K/V tile row then passes 2^32) or
                                        with (Hq/Hkv) x ceil(S/32) >= 2^31 - 16 row blocks     */
#define GQA_ATTN_ERR_UNSUPPORTED -3  /* D != 128, or a pointer that is not 16-byte aligned          */
#define GQA_ATTN_ERR_HIP         -4  /* a HIP launch or allocation failed (see gqa_attn_last_error) */
#define GQA_ATTN_ERR_WORKSPACE   -5  /* caller workspace NULL/too small, or a bad split size        */

/*
 * Causal (or full) attention over a prompt.
 *   q, out : [B, S, Hq, D]  bf16
 *   k, v   : [B, S, Hkv, D] bf16
 *   scale  : logit scale (callers normally pass 1/sqrt(D)); any finite value.
 *   causal : nonzero = query i sees keys 0..i; zero = every query sees all S keys.
 * Implements the prefill mode (chowfi/kernels README, "Result": prefill processes
 * the full prompt with a causal mask). Whole key tiles above the diagonal are
 * never visited ("What helped most", item 3), and the query tiles with the most
 * key tiles are launched first (item 4).
 * Allocates nothing.
 */
int gqa_attn_prefill(const void* q, const void* k, const void* v, void* out,
                     int B, int S, int Hq, int Hkv, int D, float scale, int causal,
                     void* stream);

/*
 * The launch gqa_attn_prefill uses for this shape. A unit is 32 query rows of
 * one head; a workgroup serves 4 or 8 units of one KV head. *key_splits is 1
 * (one wave per unit, which streams all of the unit's key tiles) or 2 (two
 * waves per unit, each streaming half of them; their softmax states are merged
 * by log-sum-exp weights before the rows are written). *waves is the workgroup
 * size in waves (units x key splits) and *workgroups the size of the grid.
 * The 8-unit form is taken once its grid holds at least 5/3 workgroups per CU;
 * the key split when the 4-unit grid holds at most 2 per CU and S >= 512.
 * For B = 1 with 32 query and 8 KV heads: S < 512 gives (4, 1),
 * 512 <= S <= 2048 gives (8, 2), S <= 3392 gives (4, 1), larger S (8, 1) as
 * (waves, key_splits). Any output may be NULL. Returns the same shape errors
 * as gqa_attn_prefill.
 */
int gqa_attn_prefill_plan(int B, int S, int Hq, int Hkv, int D, int* waves, int* workgroups,
                          int* key_splits);

/*
 * gqa_attn_prefill with the workgroup form fixed by the caller instead of chosen by
 * shape: (waves, key_splits) is one of the pairs gqa_attn_prefill_plan reports,
 * (4, 1), (8, 1) or (8, 2), or (0, 0) for the library's choice (then the call is
 * gqa_attn_prefill). Any other pair returns GQA_ATTN_ERR_UNSUPPORTED before any HIP
 * call. Every form computes the same attention: (4, 1) and (8, 1) give each wave the
 * same rows and operation order, so their outputs are identical bit for bit; (8, 2)
 * sums each row's two key halves in another order (differences of bf16 rounding
 * only). It exists for the sweep of tile shapes (every arrangement timed against
 * the others in paired rounds: "Field note 005", "The loop") and for callers that
 * want one form for every shape. Same arguments, layout, errors and asynchrony as
 * gqa_attn_prefill; allocates nothing.
 */
int gqa_attn_prefill_form(const void* q, const void* k, const void* v, void* out,
                          int B, int S, int Hq, int Hkv, int D, float scale, int causal,
                          int waves, int key_splits, void* stream);

/*
 * The prefill with the tile shape fixed by the caller, for the sweep of tile shapes
 * ("Field note 005", "The loop": the block and k-step sizes are the knobs a search
 * turns; every point timed in paired rounds against the others). A unit is 32 query
 * rows of one head; a wave owns rows_per_wave / 32 units, a workgroup `waves` waves,
 * and K/V are staged through LDS in tiles of keys_per_tile keys. Supported
 * (rows_per_wave, keys_per_tile, waves):
 *   (32, 64, 4), (32, 64, 8)   the library's own 4- and 8-wave forms (as
 *                              gqa_attn_prefill_form (4, 1) and (8, 1));
 *   (32, 32, 4), (32, 32, 8)   32-key tiles;
 *   (32, 128, 4), (32, 128, 8) 128-key tiles (the 4-wave one with 128 KB of LDS,
 *                              one workgroup per CU);
 *   (64, 32, 4), (64, 64, 4)   64 rows per wave: every K and V fragment read from LDS
 *                              feeds two units' MFMAs; one wave per SIMD.
 * Any other triple returns GQA_ATTN_ERR_UNSUPPORTED before any HIP call. Every shape
 * computes the same attention (summation order and the lazy-rescale points differ, so
 * results agree to bf16 rounding, not bit for bit). Same arguments, layout, errors and
 * asynchrony as gqa_attn_prefill; with 128-key tiles Hkv must also stay below 132105
 * (the 32-bit tile offsets). Allocates nothing.
 */
int gqa_attn_prefill_tiles(const void* q, const void* k, const void* v, void* out,
                           int B, int S, int Hq, int Hkv, int D, float scale, int causal,
                           int rows_per_wave, int keys_per_tile, int waves, void* stream);

/*
 * One-token decode against a KV cache, split along the cache.
 *   q, out         : [B, Hq, D]  bf16
 *   kcache, vcache : [B, L, Hkv, D] bf16; L is the capacity (the row stride).
 *   lens           : device int32 [B]. Sequence b attends slots 0..lens[b]-1.
 *                    Values are clamped to [0, L] in the kernel and never read
 *                    on the host. lens[b] = 0 gives a zero output row. Slots at
 *                    or past lens[b] are never read, whatever they hold.
 * Implements the decode mode ("Result": decode generates one token from a KV
 * cache of a given length). The cache is cut into nsplit splits that run in
 * parallel on all CUs and are then merged by log-sum-exp ("What helped most",
 * item 1); split s holds the 64-key tiles s, s + nsplit, s + 2 nsplit, ... of
 * the sequence, so the splits of a head read one contiguous stretch of the
 * cache at a time and a short sequence still spreads over all of them. Each
 * split's K/V rows are read once, with non-temporal loads, for all query heads
 * of their group (item 2). The merge happens in the same kernel launch (item 5,
 * one fewer launch): the last workgroup to finish a (sequence, KV head) merges
 * it, after every other split has published its partial and counted itself.
 * The split partials live in a library-owned workspace, cached per (device,
 * stream) and grown on demand: one hipMalloc (and a clear of the new buffer by a
 * small kernel on `stream`) the first time a larger size is needed, none
 * afterwards. Concurrent streams never share a workspace. A workspace that has
 * been used is never freed before gqa_attn_release: when a larger one replaces
 * it, the old one is kept (earlier work on the stream, or a graph captured from
 * it, may still use it). To capture this call into a HIP graph, make one call
 * of at least that size on the capturing stream first (a capture cannot
 * allocate), or use gqa_attn_decode_ws; the graph then uses that workspace
 * wherever it is replayed, so a replay must not overlap other decodes on that
 * stream's workspace. Calls from several host threads are safe: the workspace
 * of a stream is looked up, grown and launched on under one lock.
 */
int gqa_attn_decode(const void* q, const void* kcache, const void* vcache,
                    const int32_t* lens, void* out,
                    int B, int L, int Hq, int Hkv, int D, float scale,
                    void* stream);

/*
 * The split the library would choose for a decode of this shape.
 * On success writes the keys per split (*chunk, a multiple of 64) and the
 * number of splits (*nsplit = ceil(L / chunk)). Either output may be NULL.
 * Every decode entry point accepts at most 262144 splits (2^18) and returns
 * GQA_ATTN_ERR_WORKSPACE beyond that; the library's own choice stays within
 * it for every L up to 2^30.
 */
int gqa_attn_decode_plan(int B, int L, int Hq, int Hkv, int D, int* chunk, int* nsplit);

/*
 * Bytes of workspace a decode needs with `chunk` keys per split (0 = the
 * library's own choice). Returns 0 if the arguments are invalid.
 * Layout, each part on a 256-byte boundary: int32 counters[max(4096, B*Hq)],
 * then fp32 o_part[B][Hq][nsplit][D], then fp32 lse[B][Hq][nsplit]. The
 * counters come first and their size depends only on (B, Hq), so a zeroed
 * workspace stays valid when it is reused for other shapes.
 */
size_t gqa_attn_decode_workspace_bytes(int B, int L, int Hq, int Hkv, int D, int chunk);

/*
 * Decode with a caller-owned workspace and an explicit split size. Same
 * semantics as gqa_attn_decode, with nsplit = ceil(L / chunk) splits of about
 * chunk keys each. chunk = 0 takes the library's choice; otherwise chunk must
 * be a positive multiple of 64 with ceil(L / chunk) at most 2^18. ws must be
 * 16-byte aligned and hold at least gqa_attn_decode_workspace_bytes(..., chunk)
 * bytes.
 * The counters part of ws (its first max(4096, B*Hq) int32) must hold zeros
 * before the call: allocate the buffer zeroed; each completed call leaves the
 * counters zero again. Two calls in flight on the same workspace race.
 * Allocates nothing.
 */
int gqa_attn_decode_ws(const void* q, const void* kcache, const void* vcache,
                       const int32_t* lens, void* out,
                       int B, int L, int Hq, int Hkv, int D, float scale,
                       int chunk, void* ws, size_t ws_bytes, void* stream);

/*
 * gqa_attn_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, semantics, split and results (bit for bit) as gqa_attn_decode, but
 * the split partials and merge counters live in a fixed 8 MiB scratch array
 * that the library holds on each GPU until the process ends. The call
 * allocates nothing: it makes no hipMalloc, hipFree or other allocating call.
 * Shapes whose workspace (gqa_attn_decode_workspace_bytes with chunk 0)
 * exceeds 8 MiB are rejected with GQA_ATTN_ERR_WORKSPACE before any HIP call,
 * with the sizes in gqa_attn_last_error (with 32 query heads and 8 KV heads the
 * workspace is 0.52 MiB at batch 1 for every L up to 131072 and 4.05 MiB at
 * L = 2^20). The first call on a GPU also clears that GPU's scratch with a
 * small kernel on `stream`. Every call on one GPU shares its scratch: calls
 * that overlap in time on one GPU (other streams, other threads) race and must
 * be serialised by the caller. Device ordinals 0-63 are supported (others
 * return GQA_ATTN_ERR_HIP).
 */
int gqa_attn_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                            const int32_t* lens, void* out,
                            int B, int L, int Hq, int Hkv, int D, float scale,
                            void* stream);

/*
 * The first half of a decode on its own: per-split partial results. Here split
 * s is the contiguous chunk of cache slots [s*chunk, (s+1)*chunk), clipped to
 * lens[b] (the fused entry points above assign keys to splits differently; their
 * partials never leave the library). Writes, for every (b, h, split s):
 *   o_part[b][h][s][:] (fp32, the chunk's softmax-weighted mean of V) and
 *   lse[b][h][s]       (fp32, log2 of sum_j 2^(x_j * log2(e)) over the chunk,
 *                       i.e. the chunk's log-sum-exp in base-2 units;
 *                       -inf for an empty chunk; such a chunk's o_part row is not
 *                       written and must be ignored).
 * ws is laid out as in gqa_attn_decode_workspace_bytes (the counters are not
 * used). Allocates nothing.
 */
int gqa_attn_decode_partials(const void* q, const void* kcache, const void* vcache,
                             const int32_t* lens, int B, int L, int Hq, int Hkv, int D,
                             float scale, int chunk, void* ws, size_t ws_bytes, void* stream);

/*
 * The second half of a decode on its own: log-sum-exp merge of nsplit
 * partials (o_part then lse, laid out as above) into out [B, Hq, D] bf16.
 * A row whose every split is empty becomes zero. Allocates nothing.
 */
int gqa_attn_decode_combine(const void* ws, size_t ws_bytes, void* out,
                            int B, int Hq, int D, int nsplit, void* stream);

/*
 * Measured roofline denominators. The metakernel page ("How it works", "Return
 * schemas") derives device limits from dedicated probe kernels, each reported
 * with the clock it ran at, instead of spec-sheet figures. These two are the
 * limits of the two attention kernels. The caller times each call (for example
 * with events on `stream`); neither allocates.
 *
 * Cold HBM read rate: every byte of buf is read once with 16-byte non-temporal
 * loads (the decode kernel's width and cache policy). If bytes is a multiple of
 * 2048 and workgroups of 8, workgroup w reads the 256-byte blocks at offset
 * 256 (w mod 8) of each 2 KB row, the decode's pattern at 8 KV heads of 128
 * bf16 (lane t of workgroup w = 8k + x reads chunk t mod 16 of that block in
 * rows 16 (k + K j) + t / 16, K = workgroups / 8); otherwise lane i of the grid
 * reads the 16-byte chunks i, i + n, i + 2n, ... (n = 256 * workgroups).
 *   buf        : device, 16-byte aligned; bytes > 0 and a multiple of 16. A buffer
 *                several times the 256 MB MALL measures HBM, not the cache.
 *   workgroups : 1..65535 workgroups of 256 lanes (4096 suits MI355X).
 *   sink       : device uint32 [sink_words], sink_words >= 256 * workgroups; one
 *                XOR of the data per lane (only there so the loads are kept).
 */
int gqa_attn_probe_hbm_read(const void* buf, size_t bytes, int workgroups,
                            uint32_t* sink, size_t sink_words, void* stream);

/*
 * Register-resident bf16 MFMA rate: workgroups of 4 waves, 2 waves per SIMD,
 * each wave issuing rounds x 64 v_mfma_f32_32x32x16_bf16 (32768 flop each) on 8
 * independent fp32 accumulators, operands random bf16 (seeded) so every
 * instruction sees new data. Flops per call:
 *     workgroups * 4 * rounds * 64 * 32768.
 *   rounds     : 1..1048576;  workgroups : 1..65535 (512 = 2 per CU).
 *   sink       : device float [sink_floats], sink_floats >= 256 * workgroups.
 *   ticks      : device uint64 [ticks_count], ticks_count >= 2 * workgroups.
 *                Workgroup w writes ticks[2w] = shader-clock cycles of its MFMA
 *                loop (s_memtime) and ticks[2w+1] = the same interval in 100 MHz
 *                ticks (s_memrealtime): their ratio x 0.1 GHz is the clock it ran at.
 */
int gqa_attn_probe_mfma_bf16(int rounds, uint32_t seed, int workgroups,
                             float* sink, size_t sink_floats,
                             uint64_t* ticks, size_t ticks_count, void* stream);

/* Static description of a return code. Never NULL. */
const char* gqa_attn_strerror(int code);

/* Detail of the most recent GQA_ATTN_ERR_HIP on the calling thread ("" if none). */
const char* gqa_attn_last_error(void);

/* Frees the library-cached decode workspaces, including those replaced by larger
 * ones. The caller must ensure no decode using them is still in flight (for
 * example by synchronising the device) and that no captured graph that uses
 * them will be replayed. */
void gqa_attn_release(void);

/* ABI version of this header. */
int gqa_attn_version(void);

#define GQA_ATTN_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
