/*
 * scr.h — routed MoE over a shared expert slot cache, on MI355X (gfx950).
 *
 * C ABI of libscr.so.  Every entry point takes plain pointers and sizes and
 * enqueues its work on the caller's HIP stream; none of them allocates device
 * memory, none keeps global mutable state, and none synchronises with the host
 * except scr_stage_plan (one read-back per prefill step, by design).
 *
 * Sources (the method is described on four pull-request pages):
 *   [P1] FreeToken PR #676 "--moe-prefill-demand-tokens": a short prefill
 *        chunk routes, hands its distinct experts to the LRU slot cache one
 *        fixed-width query at a time, copies each query's misses from pinned
 *        host memory before the next query, aligns against the slot count and
 *        runs the same grouped GEMM over the slots, sized by the routed layer.
 *   [P2] gdevenyi's FreeToken PR #68: the same path, ensuring unique ids in
 *        decode-width pieces.
 *   [P3] vLLM fork PR #48 "Expert pool": one bank shared by all MoE layers,
 *        keyed (layer, expert), a device-side LRU planner, fixed-grid row
 *        copies from the host source's device-mapped view, align over logical
 *        experts with a physical-row remap, no host code between router and GEMM.
 *   [P4] vLLM fork PR #51: prefill staging into two full-layer buffers,
 *        alternating by layer, filled by DMA on a side stream while the
 *        previous layer computes; one placement read-back per step; 64-bit
 *        row offsets (the bank-size guard section).
 *
 * Conventions
 *   - "device" pointers are device memory (or device-accessible pinned host
 *     memory where stated); "host" pointers are ordinary host memory.
 *   - All arrays are owned by the caller and must stay alive until the work
 *     enqueued on the stream has finished.
 *   - Return value: SCR_OK or a negative SCR_E* code.  Arguments are checked
 *     before anything is enqueued; on error nothing is enqueued and
 *     scr_last_error() describes the failure (thread-local text).
 *   - Conditions only the device can see (a miss with no evictable slot)
 *     set bits in the bank's sticky err word; kernels never trap and never
 *     access memory outside the documented extents.
 *   - Byte offsets into banks, pools and staging buffers are 64-bit.
 */
#ifndef SCR_H_
#define SCR_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ----------------------------------------------------------------- codes */
#define SCR_OK 0
#define SCR_EINVAL (-1)     /* bad argument (null pointer, size out of range) */
#define SCR_ENOTSUP (-2)    /* unsupported dtype or shape                     */
#define SCR_ECAPACITY (-3)  /* host-detectable capacity violation             */
#define SCR_EHIP (-4)       /* HIP runtime error                              */

/* bits of the bank's sticky err word */
#define SCR_ERR_CAPACITY 1u /* a query had more misses than evictable slots */

/* weight formats */
#define SCR_W_BF16 0  /* bf16 rows                                          */
#define SCR_W_NVFP4 1 /* e2m1 codes + e4m3 per-16 block scales + fp32 global */
#define SCR_W_FP8 2   /* e4m3 codes + one fp32 scale per tensor               */
#define SCR_W_MXFP4 3 /* e2m1 codes + e8m0 per-32 block scales (OCP MX)       */
#define SCR_W_MXFP4_A8 4 /* MXFP4 records; activations as FP8 E4M3 under the layer's scales (W4A8) */
#define SCR_W_NVFP4_A4 5 /* NVFP4 records; activations as NVFP4 under the layer's scales (W4A4) */

/* output dtypes of the layer */
#define SCR_Y_F32 0
#define SCR_Y_BF16 1

/* limits */
#define SCR_MAX_TOPK 32
#define SCR_MAX_EXPERTS 4096      /* experts in one layer (route, dedup)   */
#define SCR_MAX_QUERY_WIDTH 1024  /* ids per ensure query                  */
#define SCR_MAX_SLOTS 262144      /* slots in one bank                     */
#define SCR_MAX_BUCKETS 16384     /* buckets of one align call             */

/* ------------------------------------------------------- expert record
 * One expert's weights form one contiguous record, identical in the pinned
 * host pool, in a bank slot and in a staging buffer, so a miss copy is a
 * single contiguous byte range.  Logical tensors (offsets from
 * scr_record_layout_of):
 *   SCR_W_BF16 : w13 bf16 [2I][H] (rows 0..I-1 gate, I..2I-1 up), w2 bf16 [H][I]
 *   SCR_W_NVFP4: w13 e2m1 codes [2I][H], w13 e4m3 (OCP E4M3FN) scales [2I][H/16]
 *                (one per 16 consecutive input columns of a row), w2 codes [H][I],
 *                w2 scales [H][I/16], then g13 f32, g2 f32 (global scales);
 *                record padded to 256 bytes.
 *                Decoded weight = e2m1(code) * e4m3(scale) * global.
 *   SCR_W_FP8  : w13 e4m3 (OCP E4M3FN) codes [2I][H], w2 codes [H][I], then g13
 *                f32, g2 f32 (one scale per tensor); padded to 256 bytes.
 *                Decoded weight = e4m3(code) * scale.
 *   SCR_W_MXFP4: w13 e2m1 codes [2I][H], w13 e8m0 scales [2I][H/32] (one per
 *                32 consecutive input columns of a row), w2 codes [H][I], w2
 *                scales [H][I/32]; no global scale; padded to 256 bytes.
 *                Decoded weight = e2m1(code) * 2^(scale - 127) (scale codes
 *                2..252: the products are exact bf16 values; 255 is NaN).
 * The FP8 and MXFP4 formats follow the OCP Microscaling Formats specification
 * (FreeToken PR #676, Known limits, names both for the prefill over the
 * slots without describing them; the per-tensor FP8 scale is a reading).
 * Storage is tile-major so each load of the GEMM is one contiguous range: a
 * tensor of N rows and K columns is a sequence of tile-blocks (t, kb), t over
 * the N/16 row tiles, kb over the K/128 column blocks (t-major).  Inside a
 * tile-block, with r = row % 16:
 *   bf16   4096 B: element (r, 32 s + 8 g + e) at byte 1024 s + 16 (16 g + r) + 2 e
 *   codes  1024 B: code (r, 32 g + j) in byte 16 (16 g + r) + j / 2, low nibble = even j
 *   scales  128 B: scale (r, 2 g + h) (the 16-column block 8 kb + 2 g + h) at byte
 *                  2 (16 g + r) + h
 *   fp8    2048 B: code (r, 32 g + j) at byte 1024 (j / 16) + 16 (16 g + r) + j % 16
 *   mx scales 64 B: scale (r, g) (the 32-column block 4 kb + g) at byte 16 g + r
 * H and I must be multiples of 128.
 */
typedef struct scr_record_layout {
  uint64_t w13_off, w13_scale_off, w2_off, w2_scale_off, g13_off, g2_off;
  uint64_t record_bytes;
} scr_record_layout;

int scr_record_layout_of(int wdtype, int H, int I, scr_record_layout* out);

/* --------------------------------------------------------------- bank
 * The slot cache [P1 Problem/Solution; P3 What]: S slots shared by L layers
 * of E experts, keyed key = layer * E + expert.  All pointers are device.
 *   slot_key    int32  [S]    key held by the slot, -1 = empty
 *   slot_stamp  uint64 [S]    recency stamp of the slot, 0 = never used
 *   key_to_slot int32  [L*E]  slot holding the key, -1 = not resident
 *   clock       uint64 [1]    ticks once per ensure query
 *   stats       uint64 [4]    hits, misses, evictions, queries (decode only)
 *   decode_freq uint32 [L*E]  per-key routed count (decode only)
 *   err         uint32 [1]    sticky SCR_ERR_* bits
 *   rows        uint8  [S * record_bytes]  the slots' expert records
 * slot_key and key_to_slot are kept inverse to each other by every call.
 * Eviction policy (policy):
 *   SCR_POLICY_LRU  victims in ascending (stamp, slot) among the slots the
 *                   query did not touch [P1 author's reply: LRU only].
 *   SCR_POLICY_LRFU scored eviction [P1 run notes: the author's build admits
 *                   by LRFU; P1 Solution: earlier pieces pinned against later
 *                   ones].  Per slot a combined recency-frequency value
 *                   C = sum over its references of 2^-(lambda * age), kept in
 *                   slot_crf as unsigned Q8.24 at the slot's stamp; lrfu_decay
 *                   = D = 2^32 * 2^-lambda (0 < D < 2^32) is the per-tick
 *                   factor.  D^n is r = 2^32, b = D, for each bit of n from the
 *                   lowest: r = r * b >> 32 if set, b = b * b >> 32;
 *                   decay(C, n) = C * r >> 32.  A hit sets C = min(decay(C,
 *                   now - stamp) + 2^24, 2^32 - 1), an admission C = 2^24.
 *                   Victims in ascending (decay(C, now - stamp), slot) among
 *                   the slots untouched by the whole chunk: stamp below
 *                   *chunk_start, the clock of the chunk's first query (set by
 *                   scr_ensure_slots at q_begin = 0 and by the batched and
 *                   one-launch planners).
 *   slot_crf    uint32 [S]  LRFU only (may be NULL under LRU)
 *   chunk_start uint64 [1]  LRFU only (may be NULL under LRU)
 */
#define SCR_POLICY_LRU 0
#define SCR_POLICY_LRFU 1
typedef struct scr_bank_desc {
  int32_t S, L, E, wdtype;
  int32_t* slot_key;
  uint64_t* slot_stamp;
  int32_t* key_to_slot;
  uint64_t* clock;
  uint64_t* stats;
  uint32_t* decode_freq;
  uint32_t* err;
  uint8_t* rows;
  uint64_t record_bytes;
  int32_t policy;
  uint32_t lrfu_decay;
  uint32_t* slot_crf;
  uint64_t* chunk_start;
} scr_bank_desc;

/* ---------------------------------------------------------- host pool
 * The pinned host source of every copy [P3 What; P4 Prefill staging].
 *   key_rows_dev  device [L*E]: device-accessible addresses (the device-mapped
 *                 view of pinned memory) of each key's record, read by kernels;
 *   key_rows_host host   [L*E]: the same records' host addresses (stage_plan
 *                 merges host-adjacent records into runs with them).
 * Several keys may share one record (payload aliasing); records are 16-byte
 * aligned and record_bytes is a multiple of 16.
 */
typedef struct scr_host_pool {
  int32_t L, E;
  const void* const* key_rows_dev;
  const void* const* key_rows_host;
  uint64_t record_bytes;
} scr_host_pool;

/* ------------------------------------------------------- routed view
 * RoutedExperts [P1 Solution, fourth bullet]: the routed layer's expert count
 * and input scales travel beside the bucket range, so tiles and scales come
 * from the layer, never from the bank.
 *   bucket_rows       device [num_buckets]: record address of each bucket (a
 *                     slot of the bank, an expert of a streamed layer buffer,
 *                     or a row of a staging buffer); entries of buckets never
 *                     routed to are not read.
 *   input_scale       device [num_experts]: the layer's per-expert scales of
 *                     the gate/up input x, indexed by logical expert.
 *   down_input_scale  device [num_experts]: the same for the down input h;
 *                     may be NULL except for the activation-quantising
 *                     formats (SCR_W_MXFP4_A8, SCR_W_NVFP4_A4).
 *   The activation-quantising formats divide by the maxima of these arrays:
 *   they must hold positive finite values (device data: not checked).
 */
typedef struct scr_routed_experts {
  int32_t layer, num_experts, k, H, I, wdtype, num_buckets;
  const void* const* bucket_rows;
  const float* input_scale;
  const float* down_input_scale;
} scr_routed_experts;

/* tile configuration of the grouped GEMM; a function of (T, k, E_layer,
 * wdtype) only [P1 Solution: tiles from tokens per expert of the routed layer] */
typedef struct scr_tile_cfg {
  int32_t block_m;   /* align block size (rows of one MFMA M tile)      */
  int32_t m_chunk;   /* rows one workgroup holds per pass over a bucket */
  int32_t n_tile_gu; /* h columns per gate/up workgroup (per N chunk for
                        the 112-row kernels, whose workgroups take one or
                        more chunks)                                     */
  int32_t n_tile_dn; /* output columns per down workgroup (likewise)     */
  int32_t wdtype;
} scr_tile_cfg;

/* staging run: experts [e_begin, e_begin + count) of one layer, contiguous in
 * the host pool and in the staging buffer */
typedef struct scr_run {
  int32_t layer, e_begin, count;
} scr_run;

/* ======================================================= entry points */

/* route [P1 Known limits; P2 commit 1: route, then fetch the missing routed
 * experts, then the slot GEMM].  Per token, the k largest logits in
 * descending order (ties: lower expert id) and their softmax weights: the
 * softmax of the k selected logits, evaluated in fp64 and rounded once to fp32.
 *   logits   device f32 [T][E] row-major      topk_ids device i32 [T][k]
 *   topk_w   device f32 [T][k]
 * 1 <= k <= min(E, SCR_MAX_TOPK), 1 <= E <= SCR_MAX_EXPERTS, T >= 0 (T = 0 is a no-op).
 * Logits must not be NaN. */
int scr_route(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
              hipStream_t stream);

/* dedup [P1 Solution, second bullet; P1 gdevenyi comment].  The distinct
 * expert ids of ids[0..n) ascending, as a list of fixed length Lmax = min(n, E)
 * padded with the sentinel E, so the host knows its length without a sync.
 *   ids        device i32 [n]; entries outside [0, E) are ignored
 *   distinct   device i32 [Lmax]
 *   n_distinct device i32 [1]
 *   inverse    device i32 [n] or NULL: index into distinct of ids[i] (-1 if ignored)
 * 1 <= E <= 8192, n >= 0. */
int scr_dedup(const int32_t* ids, int n, int E, int32_t* distinct, int32_t* n_distinct,
              int32_t* inverse, hipStream_t stream);

/* ensure_slots [P1 Solution second bullet, author's reply; P3 What].  One LRU
 * query: the ids distinct[q_begin .. q_begin + width) of `layer`.  The clock
 * ticks once; hits get the new stamp; misses, in query order, take the slots
 * not stamped by this query in ascending (stamp, slot) order (empty slots have
 * stamp 0); an evicted key is unmapped.  The admitted misses are listed for
 * scr_copy_misses.  record_stats = 0 (prefill) leaves stats and decode_freq
 * untouched; recency still moves.  Misses beyond the evictable slots set
 * SCR_ERR_CAPACITY in bank->err and are not admitted.
 *   distinct  device i32, entries outside [0, E) are skipped; the valid
 *             entries of one query must be distinct
 *   miss_slot, miss_key device i32 [width]; n_miss device i32 [1]
 * 1 <= width <= SCR_MAX_QUERY_WIDTH, 0 <= layer < L, bank->S <= SCR_MAX_SLOTS. */
int scr_ensure_slots(const scr_bank_desc* bank, int layer, const int32_t* distinct, int q_begin,
                     int width, int record_stats, int32_t* miss_slot, int32_t* miss_key,
                     int32_t* n_miss, hipStream_t stream);

/* ensure_slots_batched [P1 Solution second bullet and the author's reply].
 * The queries distinct[i*width .. i*width + width) for i < ceil(n / width), in
 * order, in one launch; each is exactly one scr_ensure_slots call (its own
 * clock tick, same slot decisions).  n_miss[i] receives query i's admitted
 * count; the admitted misses of all queries are appended to miss_slot /
 * miss_key, *n_total of them.  An entry whose slot a later query of the same
 * call took again is marked superseded (slot -1), so one scr_copy_misses over
 * the list (max_miss = n) moves each slot's final record.  Under LRU with
 * min(T*k, E) <= S no query evicts an earlier query's admission (LRU evicts
 * them last), so this equals copying each query's misses before the next.
 *   n_miss device i32 [ceil(n / width)], miss_slot/miss_key device i32 [n],
 *   n_total device i32 [1]; 1 <= width <= SCR_MAX_QUERY_WIDTH, n >= 1. */
int scr_ensure_slots_batched(const scr_bank_desc* bank, int layer, const int32_t* distinct, int n,
                             int width, int record_stats, int32_t* miss_slot, int32_t* miss_key,
                             int32_t* n_miss, int32_t* n_total, hipStream_t stream);

/* plan_chunk [P1 Solution bullets 2-3: the distinct list, then the LRU
 * queries of fixed width; P3 What: a device-side planner; P1 Tests: align of
 * the routes by their slots].  The chunk's whole planning in one launch (one
 * workgroup): exactly scr_dedup(ids, n, E, distinct, n_distinct, NULL), then
 * scr_ensure_slots_batched(bank, layer, distinct, min(n, E), width, ...), then
 * scr_align_blocks(ids, n, key_to_slot + layer * E, E, S, block_size, ...),
 * with the same outputs, bank updates and error bit.  The caller then copies
 * the final misses with one scr_copy_misses over n_total.
 *   ids         device i32 [n] routed expert ids of the layer (route r = t*k+j)
 *   distinct    device i32 [min(n, E)], n_distinct device i32 [1]
 *   miss_slot, miss_key device i32 [min(n, E)]; n_miss device i32
 *               [ceil(min(n, E) / width)]; n_total device i32 [1]
 *   sorted_routes .. n_active: as scr_align_blocks with num_buckets = S
 * Returns SCR_ENOTSUP (nothing launched) when n > 4096, E > 8192 or S > 8192,
 * where the separate calls apply. */
int scr_plan_chunk(const scr_bank_desc* bank, int layer, const int32_t* ids, int n, int32_t* distinct,
                   int32_t* n_distinct, int width, int record_stats, int32_t* miss_slot, int32_t* miss_key,
                   int32_t* n_miss, int32_t* n_total, int block_size, int32_t* sorted_routes,
                   int32_t* block_bucket, int32_t* n_post_pad, int32_t* active_buckets,
                   int32_t* active_block_begin, int32_t* n_active, hipStream_t stream);

/* copy_misses [P1 Solution second bullet; P3 What: fixed-grid row copies from
 * the host source's device-mapped view].  For i < *n_miss (read on the
 * device) copies the record of key miss_key[i] from the pool into bank slot
 * miss_slot[i].  The grid depends only on max_miss, not on *n_miss, so the
 * call needs no host sync.  pool->record_bytes must equal bank->record_bytes.
 * Entries with miss_slot < 0 are skipped.  0 <= *n_miss <= max_miss <= 65536. */
int scr_copy_misses(const scr_bank_desc* bank, const scr_host_pool* pool, const int32_t* miss_slot,
                    const int32_t* miss_key, const int32_t* n_miss, int max_miss,
                    hipStream_t stream);

/* align_blocks [P1 Solution third bullet and Tests; P1 gdevenyi comment;
 * P3 What: align over logical experts ignoring invalid ones].
 * bucket(r) = id_to_bucket ? id_to_bucket[ids[r]] : ids[r]; routes whose id is
 * outside [0, num_ids) (with a map) or whose bucket is outside [0, num_buckets)
 * are dropped.  Buckets are laid out in ascending order, each holding its
 * routes in ascending route index, padded with the sentinel n to a multiple of
 * block_size.  No limit on num_buckets beyond SCR_MAX_BUCKETS (multi-workgroup).
 *   sorted_routes      device i32 [cap]      cap = scr_align_capacity(n, num_buckets, block_size)
 *   block_bucket       device i32 [cap / block_size]  bucket of each block, -1 past the end
 *   n_post_pad         device i32 [1]        padded total (multiple of block_size)
 *   active_buckets     device i32 [min(n, num_buckets)]  non-empty buckets, ascending
 *   active_block_begin device i32 [min(n, num_buckets) + 1]  first block of each; the
 *                      entry after the last active bucket is n_post_pad / block_size
 *   n_active           device i32 [1]
 *   ws                 device scratch of scr_align_workspace(...) bytes
 * block_size in {16, 32, 64}; 0 <= n < 2^30. */
size_t scr_align_capacity(int n, int num_buckets, int block_size);
int scr_align_workspace(int n, int num_buckets, size_t* bytes);
int scr_align_blocks(const int32_t* ids, int n, const int32_t* id_to_bucket, int num_ids,
                     int num_buckets, int block_size, int32_t* sorted_routes,
                     int32_t* block_bucket, int32_t* n_post_pad, int32_t* active_buckets,
                     int32_t* active_block_begin, int32_t* n_active, void* ws, size_t ws_bytes,
                     hipStream_t stream);
/* align_blocks_noalloc: for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  scr_align_blocks with the same arguments except the
 * workspace, and the same outputs.  Its scratch is a file-scope device array
 * of the library, 4,325,632 bytes on each GPU it runs on, held until the
 * process ends; the call allocates nothing.  All calls on one GPU share that
 * GPU's array, so calls that overlap on one GPU (several streams or threads)
 * race: the caller serialises them.  Every scratch entry a call reads is
 * written earlier in the same call, so nothing carries over between calls.
 * SCR_ECAPACITY if a shape needs more scratch than the array holds (none
 * with num_buckets <= SCR_MAX_BUCKETS does). */
int scr_align_blocks_noalloc(const int32_t* ids, int n, const int32_t* id_to_bucket, int num_ids,
                             int num_buckets, int block_size, int32_t* sorted_routes,
                             int32_t* block_bucket, int32_t* n_post_pad, int32_t* active_buckets,
                             int32_t* active_block_begin, int32_t* n_active, hipStream_t stream);

/* tile config [P1 Solution fourth bullet, Tests: tiles sized by the routed
 * layer's experts, never by the slot count]. */
int scr_tile_config(int T, int k, int E_layer, int wdtype, scr_tile_cfg* cfg);
/* workspace of scr_grouped_moe_forward: h [cap][I] bf16 + per-route rows [T*k][H]
 * (fp32 for bf16 weights when cfg->m_chunk is 32 or the shape is one the
 * long-chunk kernels do not take; otherwise fp16 values times 2^e with one
 * int8 e per 32 columns, [T*k][H/32] after the rows) + per-route flags + the
 * two activation scales; SCR_W_MXFP4_A8 holds the E4M3 codes of x [T][H] and
 * of h [cap][I] in place of h; SCR_W_NVFP4_A4 the decoded NVFP4 values of x
 * [T][H] and of h [cap][I] as fp16; SCR_W_NVFP4 also an fp16 copy of x [T][H]
 * and its row exponents [T] */
int scr_moe_workspace(int T, int k, int E_layer, int H, int I, const scr_tile_cfg* cfg,
                      size_t* bytes);

/* grouped_moe_forward [P1 Solution: the same grouped GEMM over the layer's
 * slots; P4 Root cause: weights read once per slot, not once per M block].
 * For every active bucket (from scr_align_blocks): gate/up GEMM with SwiGLU,
 * then the down GEMM scaled by each route's weight, then
 *   y[t] = sum_{j < k} w[t][j] * W2_e (silu(G_e x_t) * (U_e x_t)),  summed in rank order j.
 * The grid is bounded by min(T*k, view->num_experts) active buckets, a layer
 * size, never a bank size.
 *   x           device bf16 [T][H]
 *   topk_w      device f32 [T][k]   (route r = t*k + j)
 *   sorted_routes, active_buckets, active_block_begin, n_active: align outputs
 *               computed with block_size = cfg.block_m over view->num_buckets
 *   y           device [T][H], f32 or bf16 per y_dtype
 *   ws          device scratch of scr_moe_workspace(...) bytes
 *   cfg_out     host, nullable: receives the tile config used
 *   a_scale_out device f32 [2], nullable: the layer's activation scales, the
 *               max of view->input_scale and the max of view->down_input_scale
 *               (0 when that is NULL) [P1 Solution, fourth bullet]
 *   marks       host array of 5 events or NULL: recorded on `stream` before
 *               the launches, again before gate/up (marks 0 and 1 bracket the
 *               activation quantisation of the A8/A4 formats and nothing
 *               otherwise: the gate/up kernel itself clears the per-route
 *               flags and reports a_scale), and after the gate/up, down and
 *               combine kernels (per-kernel timing on the launching stream);
 *               NULL entries are skipped
 * H % 128 == 0, I % 128 == 0, 128 <= H, I <= 16384 (the GEMM's K block is 128).
 * Activation-quantising formats [P1 Solution, fourth bullet; Tests, fourth
 * bullet: the activations are quantised under the max of the routed layer's
 * input scales, never the bank's]: a1 = max(input_scale[0..E)),
 * a2 = max(down_input_scale[0..E)).
 *   SCR_W_MXFP4_A8 (W4A8): x as E4M3 codes of x / a1 (scr_quantize_fp8's rule),
 *     each route's h as E4M3 codes of h / a2 (computed from the fp32
 *     accumulators), both GEMMs on the block-scaled fp8 x fp4 MFMA with unit
 *     activation scales and a1 (a2) applied to the fp32 accumulators.
 *   SCR_W_NVFP4_A4 (W4A4): x and h as NVFP4 with a1 (a2) as global scale
 *     (scr_quantize_nvfp4's rule; h per route and 16 columns); activation and
 *     weight codes times their block scales are exact fp16 values, so both
 *     GEMMs run on the fp16 MFMA over exact operands, the global scales applied
 *     to the fp32 accumulators.
 *   Both need down_input_scale, H a multiple of 512 and I a multiple of 256
 *   (SCR_ENOTSUP otherwise, nothing launched).
 * SCR_W_NVFP4 with many rows per expert (the wide kernels: cfg.m_chunk 112,
 * H a multiple of 512 and I of 256): the gate/up runs on the fp16 MFMA.  Between
 * marks 1 and 2 (so inside the gate/up time) each row of x is copied to
 * fp16 times 2^e, e putting the row's largest magnitude in [2^14, 2^15); the
 * weights decode exactly to fp16 (e2m1 times e4m3 fits), and the fp32
 * accumulators are multiplied by 2^-e after the global scale.  The products
 * and sums are those of the bf16 values, except that elements below 2^-28
 * of their row's largest magnitude round as fp16 subnormals. */
int scr_grouped_moe_forward(const scr_routed_experts* view, const void* x, int T,
                            const float* topk_w, const int32_t* sorted_routes,
                            const int32_t* active_buckets, const int32_t* active_block_begin,
                            const int32_t* n_active, void* y, int y_dtype, void* ws,
                            size_t ws_bytes, scr_tile_cfg* cfg_out, float* a_scale_out,
                            hipEvent_t* marks, hipStream_t stream);

/* quantize_fp8 [P1 Solution, fourth bullet: activations quantised under the
 * max of the layer's input scales; the static FP8 activation encoding is a
 * reading]: with a = max(scales[0..n_scales)) (device f32) and r = 1 / a (an
 * IEEE fp32 division), codes[i] = the OCP E4M3FN code of the fp32 product
 * x[i] * r, rounded to nearest even and saturated to +-448.  x device bf16 [rows][cols], codes device u8
 * [rows][cols].  Inputs finite, a > 0. */
int scr_quantize_fp8(const void* x, long long rows, int cols, const float* scales, int n_scales,
                     uint8_t* codes, hipStream_t stream);

/* quantize_nvfp4 [same passage; NVFP4 activations with the layer scale as
 * their global scale]: with a = max(scales[0..n_scales)), per row and block
 * of 16 consecutive columns: block = E4M3 code of amax / (6 * a) (fp32
 * product and division, nearest even, saturated to 448), then per element
 * the E2M1 code of the fp32 product x * r, r = 1 / (e4m3(block) * a) (one
 * IEEE division per block; nearest, ties to even, saturated to +-6; sign bit
 * set for every negative input); a block whose scale is zero gets zero
 * codes.  x device bf16 [rows][cols], cols a multiple of 16;
 * codes device u8 [rows][cols / 2] (low nibble = even column); block_scales
 * device u8 [rows][cols / 16].  Inputs finite, a > 0. */
int scr_quantize_nvfp4(const void* x, long long rows, int cols, const float* scales, int n_scales,
                       uint8_t* codes, uint8_t* block_scales, hipStream_t stream);

/* ------------------------------------------------ whole-layer / staging */

/* stream_layer_async [P1 Problem: the streamed path copies every expert of the
 * layer].  Copies the records of experts 0..E-1 of `layer` from the pool into
 * dst (device, E * record_bytes), expert e at e * record_bytes, on `stream`:
 * a copy kernel reads each record through key_rows_dev (the pinned pool's
 * device-mapped view; about 57 GB/s over PCIe 5 against about 50 for DMA). */
int scr_stream_layer_async(const scr_host_pool* pool, int layer, void* dst, hipStream_t stream);

/* stage_plan [P4 Details, prefill staging: residency changes only during
 * decode, so one read-back at the start of a prefill step serves all of its
 * layers; absent experts are grouped into contiguous runs].  Reads key_to_slot of
 * layers [layer_begin, layer_begin + n_layers) into host_map (host i32
 * [n_layers * E]), synchronising `stream` (the step's one host sync), and
 * writes the runs of non-resident experts whose host records are adjacent
 * into runs (host, capacity max_runs), layer by layer, ascending.
 * *n_runs receives the count; SCR_ECAPACITY if max_runs is too small. */
int scr_stage_plan(const scr_bank_desc* bank, const scr_host_pool* pool, int layer_begin,
                   int n_layers, int32_t* host_map, scr_run* runs, int max_runs, int* n_runs,
                   hipStream_t stream);

/* stage_rows_async [P4 Prefill staging: copies from the pinned source on a
 * side stream, layer i+1 while layer i computes, ordered with events].  On
 * `side`: waits for wait_on (nullable), copies every run of `layer` in
 * runs[0..n_runs) into dst_layer_buf at e * record_bytes, then records `done`
 * (nullable).  The copy is a kernel of 64 workgroups reading each record
 * through key_rows_dev (the pages' design uses DMA; the kernel sustains about
 * 57 GB/s against about 50 and leaves most CUs to the GEMM on the other
 * stream); the run list travels as kernel arguments, 240 runs per launch. */
int scr_stage_rows_async(const scr_host_pool* pool, const scr_run* runs, int n_runs, int layer,
                         void* dst_layer_buf, hipStream_t side, hipEvent_t wait_on,
                         hipEvent_t done);
/* stage_rows_dma_async [P4 Prefill staging, in the pages' form: one
 * hipMemcpyAsync per run from the pinned source on the side stream].  The
 * same arguments, ordering and result as scr_stage_rows_async; each run's
 * host records must be adjacent (scr_stage_plan builds runs so; SCR_EINVAL
 * otherwise, nothing enqueued).  Uses key_rows_host. */
int scr_stage_rows_dma_async(const scr_host_pool* pool, const scr_run* runs, int n_runs, int layer,
                             void* dst_layer_buf, hipStream_t side, hipEvent_t wait_on,
                             hipEvent_t done);

/* ------------------------------------------------------------ helpers */

/* bucket_rows[i] = base + i * stride for i < n (a bank's slots, or a streamed
 * layer buffer's experts). */
int scr_fill_row_table(const void* base, int n, uint64_t stride, const void** bucket_rows,
                       hipStream_t stream);
/* bucket_rows[e] = bank slot record if key (layer, e) is resident, else
 * staging + e * record_bytes: the staged view of one layer [P4 Prefill staging:
 * the staging buffer replaces the host view as the source of non-resident rows]. */
int scr_fill_staged_rows(const scr_bank_desc* bank, int layer, const void* staging,
                         const void** bucket_rows, hipStream_t stream);
/* rebuilds key_to_slot from slot_key (all keys -1, then one entry per used
 * slot); use after writing an initial slot_key/slot_stamp/clock. */
int scr_bank_rebuild_map(const scr_bank_desc* bank, hipStream_t stream);
/* bank_init [P3 What: one bank of (layer, expert) keys shared by every layer;
 * P1 Tests: the layer-view test starts from a bank that decode already filled
 * with other layers' experts].  Sets the bank's replacement state from host
 * arrays: slot_key <- host_slot_keys [S] (-1 = empty, else a key in [0, L*E)
 * held by no other slot), slot_stamp <- host_stamps [S] (none above clock; 0
 * for an empty slot), the clock <- clock; clears stats, decode_freq, err and,
 * when present, slot_crf and chunk_start; rebuilds key_to_slot.  Slot records
 * (rows) are left as they are.  An initialisation helper: the copies are
 * enqueued on `stream`, which is synchronised before the call returns, so
 * the host arrays may be freed at once.  A state that breaks the rules above
 * returns SCR_EINVAL with nothing enqueued. */
int scr_bank_init(const scr_bank_desc* bank, const int32_t* host_slot_keys, const uint64_t* host_stamps,
                  uint64_t clock, hipStream_t stream);
/* device-accessible alias of a pinned host address */
int scr_host_device_alias(const void* host_ptr, void** dev_ptr);

/* demand dispatch [P1 Solution, Tests]: threshold 0 = never; else T <= threshold */
int scr_prefill_on_demand(int T, int threshold);
/* capacity guard [P1 author's reply; P2 commit 2]: min(T*k, E) <= S (or <= S/2) */
int scr_demand_capacity_ok(int T, int k, int E, int S, int half);

/* timing events for per-kernel measurement on the launching stream: created
 * with hipEventDisableSystemFence, so recording one between kernels costs no
 * cache write-back.  elapsed waits for `stop`, then reports stop - start in ms. */
int scr_timer_create(hipEvent_t* ev);
int scr_timer_record(hipEvent_t ev, hipStream_t stream);
int scr_timer_elapsed_ms(hipEvent_t start, hipEvent_t stop, float* ms);
int scr_timer_destroy(hipEvent_t ev);

const char* scr_last_error(void);
const char* scr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SCR_H_ */
