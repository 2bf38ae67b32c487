/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged FP8-KV attention library.
 *
 * One operation: attention of new query tokens over a KV cache that is kept
 * in fixed-size pages of a preallocated pool, stored as FP8 E4M3 bytes with
 * one fp32 scale per (page, kv head), with grouped/multi-query heads; and
 * the steps on either side of it: appending new tokens' K/V to the pool,
 * and greedy acceptance of MTP drafts after verification.
 *
 * The operation follows these passages:
 *   - Atlas engine article (ainews.cool), section "技术深度解析":
 *       memory architecture -- KV cache in fixed-size blocks preallocated from
 *         a pool, no allocation while serving (hence the plan object, which
 *         allocates its workspace once, and the allocation-free forward);
 *       attention -- a FlashAttention-2 variant with tiling chosen per
 *         sequence length and GPU, and dedicated MQA/GQA kernels;
 *       quantisation -- FP8 with per-group scale factors fused into kernels.
 *   - "Atlas Takes On vLLM With a Pure Rust/CUDA Inference Engine on a
 *     Single GB10" (ainews.surl.tw): a paged FP8 KV cache; multi-token
 *     prediction with K=4 draft tokens, whose verification is attention of
 *     1+K causal query tokens per sequence.
 *
 * Result (exact arithmetic): for sequence b with L_b keys and Q_b new query
 * tokens, new token i (0-based) and query head hq,
 *     h      = hq / (Hq / Hkv)                       (kv head of the group)
 *     K~[t]  = dec(k byte of token t, head h) * kv_scales[0][page(t)][h]
 *     V~[t]  = dec(v byte of token t, head h) * kv_scales[1][page(t)][h]
 *     z_t    = sm_scale * <q[r_b+i][hq][:], K~[t]>   for t <= L_b - Q_b + i
 *     out[r_b+i][hq][:] = sum_t softmax(z)_t * V~[t]
 * where r_b = Q_0 + ... + Q_{b-1} and page(t) = block_table[b][t / 16].
 *
 * Memory layouts (all buffers are device memory, caller-owned):
 *   q           [sum Q_b][Hq][D]  ATTN_DTYPE_BF16 or ATTN_DTYPE_F32
 *   k_pages     uint8 [P][Hkv][D/16][16][16] inside a (page, head): 16-byte
 *               blocks of d, slot-major within a block; the byte of slot s,
 *               dim d sits at ((d/16)*16 + s)*16 + d%16
 *   v_pages     uint8 [P][Hkv][4][D/64][16][4][4] inside a (page, head): four
 *               consecutive slots interleaved per d; with NVB = D/16 and
 *               d = NVB*a + 4*i + e, the byte of slot s, dim d sits at
 *               ((((s/4)*(D/64) + i)*16 + a)*4 + e)*4 + s%4
 *   kv_scales   fp32  [2][P][Hkv]            [0] K scales, [1] V scales
 *   block_table int32 [B][max_pages_per_seq] physical page ids
 *   ctx_lens    int32 [B]   L_b (counts the Q_b new tokens, whose K/V are
 *                            already in the pages)
 *   q_lens      int32 [B]   Q_b
 *   out         [sum Q_b][Hq][D]  ATTN_DTYPE_BF16 (round to nearest even)
 *               or ATTN_DTYPE_F32
 * dec() is the OCP 8-bit floating point E4M3 format (bias 7, max 448, NaN
 * only at 0x7F/0xFF) by default, or a signed INT8 (desc.kv_format).
 *
 * Device-data preconditions (not checked on the hot path; breaking one is
 * undefined and may fault):
 *   1 <= Q_b <= max_q_len, Q_b <= L_b <= max_ctx_len;
 *   block_table[b][j] in [0, P) for j < ceil(L_b / 16);
 *   the K/V bytes of tokens t < L_b are not NaN codes.
 * Entries of block_table past ceil(L_b/16), bytes of slots >= L_b in the last
 * page and every unreferenced page are never used (they may hold anything).
 *
 * Errors: every entry point returns an attn_status_t.  Host-checkable
 * problems (null or misaligned pointers, bad descriptor) return before any
 * device work is enqueued.  A failed HIP call returns ATTN_ERR_HIP; the HIP
 * error code is then available from attn_last_hip_error() on that thread.
 *
 * Threading: a plan may be used by one stream at a time (its workspace is
 * shared by the forwards it enqueues); distinct plans are independent.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct attn_plan_s* attn_plan_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, inconsistent descriptor */
  ATTN_ERR_UNSUPPORTED = 2,      /* valid request this library does not implement */
  ATTN_ERR_OUT_OF_MEMORY = 3,    /* workspace allocation failed */
  ATTN_ERR_HIP = 4               /* a HIP runtime call failed */
} attn_status_t;

typedef enum { ATTN_DTYPE_F32 = 0, ATTN_DTYPE_BF16 = 1 } attn_dtype_t;

/* Format of the K/V bytes in the pages.  The quantisation section of the
 * Atlas article lists INT4/INT8/FP8 with per-group scales; with ATTN_KV_INT8
 * a byte is a two's-complement integer in [-128, 127] and its value is that
 * integer times the page's scale (the same scales, layouts and rules as
 * E4M3 otherwise).  INT8 plans take BF16 q and out; attn_kv_append on an
 * INT8 plan uses 127 in place of 448 and the integer nearest to
 * value / scale (ties to even, clipped to +-127).
 * With ATTN_KV_INT4 (head_dim 128, BF16 q and out) every byte holds two
 * 4-bit two's-complement codes in [-8, 7], code j of a byte in bits 4j..4j+3,
 * and a value is its code times the page's scale; a (page, kv head) chunk is
 * 1 KB of K and 1 KB of V:
 *   k_pages  uint8 [P][Hkv][4][16][D/8]: with u = d % 32, the K code of
 *            slot s, dim d is code u % 2 of byte [d / 32][s][u / 2]
 *   v_pages  uint8 [P][Hkv][4][16][D/16][2]: with d = (D/16)*a + r, the V
 *            code of slot s, dim d is code s % 2 of byte [s / 4][a][r][(s % 4) / 2]
 * (16 consecutive bytes hold one lane's MFMA operand codes).
 * attn_kv_append does not write INT4 pools (ATTN_ERR_UNSUPPORTED). */
typedef enum { ATTN_KV_E4M3 = 0, ATTN_KV_INT8 = 1, ATTN_KV_INT4 = 2 } attn_kv_format_t;

/* Static shape of the work a plan serves (the "adaptive tiling" of the
 * attention section: tile and split sizes are chosen from it once). */
typedef struct {
  int32_t num_seqs;          /* B >= 1 */
  int32_t num_q_heads;       /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;      /* Hkv >= 1 */
  int32_t head_dim;          /* D: 64 or 128 */
  int32_t page_size;         /* S: 16 */
  int32_t num_pages;         /* P: pages in the pool */
  int32_t max_pages_per_seq; /* row stride of block_table, >= ceil(max_ctx_len/16) */
  int32_t max_q_len;         /* bound on every Q_b, >= 1 */
  int32_t max_ctx_len;       /* bound on every L_b, >= max_q_len */
  attn_dtype_t q_dtype;      /* BF16 or F32 */
  attn_dtype_t out_dtype;    /* BF16 or F32 */
  float sm_scale;            /* softmax scale; 0 means 1/sqrt(head_dim) */
  int32_t num_kv_splits;     /* 0: plan chooses; n >= 1: the keys of all
                                (sequence, kv head, column block) segments are
                                cut into segments * n equal contiguous
                                partitions (so each of equal-length segments
                                gets exactly n), merged by log-sum-exp */
  int32_t kv_format;         /* ATTN_KV_E4M3 (0), ATTN_KV_INT8 (1) or ATTN_KV_INT4 (2) */
  int32_t kv_piece_len;      /* 0: off.  k = 32 times a power of two, with
                                num_kv_splits 0: batch-invariant split.  The
                                keys of every segment are cut every k keys
                                from its first key; each piece is computed on
                                its own and the pieces of a segment are merged
                                in an order fixed by their count.  A sequence's
                                output then depends only on its own q, lengths
                                and pages, not on the other sequences, num_seqs
                                or max_ctx_len, among plans with the same
                                heads, head_dim, max_q_len, dtypes, kv_format
                                and kv_piece_len (bit-identical rows).  The
                                workspace holds one partial per piece:
                                segments * ceil(ceil(max_ctx_len/32) / (k/32))
                                of them.  Any other value: INVALID_ARGUMENT. */
  int32_t reserved[2];       /* must be zero */
} attn_plan_desc_t;

/* What the plan chose (for tests and measurement).  A segment is one
 * (sequence, kv head, block of query columns) with the keys its columns see,
 * cut into 32-key chunks; the chunks of all segments, laid end to end, are
 * shared equally by the work units of the attention kernel (its waves in the
 * packed layout, its workgroups otherwise). */
typedef struct {
  int32_t col_tiles;              /* 16-column MFMA tiles per wave (1 or 2) */
  int32_t dup_lo_columns;         /* 1: low parts of P ride in spare MFMA columns */
  int32_t cols_per_block;         /* query columns (token x head of a group) per segment */
  int32_t col_blocks;             /* segments along the query columns of a group */
  int32_t waves_per_group;        /* waves per workgroup */
  int32_t num_segments;           /* B * Hkv * col_blocks */
  int32_t grid_size;              /* workgroups of the attention kernel */
  int32_t merge_grid_size;        /* merge kernel workgroups along x, one per segment
                                     (0: not launched); along y one per slice of the
                                     block's columns: single columns for blocks of at
                                     most 4 columns or with many pieces per segment,
                                     else up to 1024 / head_dim columns */
  int32_t work_units;             /* units sharing the chunks at most: waves when packed,
                                     workgroups otherwise */
  int32_t packed;                 /* > 0: at most 4 query columns, four pages per score
                                     tile, one wave per chunk range, this many groups
                                     of four pages in flight per wave (1 or 2) */
  int32_t shared_kv;              /* 1: more than 16 query columns; the waves of a
                                     workgroup split the columns and share each KV
                                     chunk through LDS */
  int32_t resident_groups_per_cu; /* attention workgroups one compute unit holds at once */
  int32_t compute_units;          /* of the plan's device */
  size_t workspace_bytes;         /* device bytes owned by the plan */
  int32_t wallclock_khz;          /* rate of the counter attn_plan_set_timeline records */
} attn_plan_info_t;

/* Validate desc, choose tiles/splits, allocate the workspace once with
 * hipMalloc on the current device.  On success *plan owns that memory.
 * No device work is enqueued. */
attn_status_t attn_plan_create(const attn_plan_desc_t* desc, attn_plan_t* plan);

/* Enqueue the attention on `stream` (asynchronous: no allocation, no host
 * synchronisation).  Pointers are device pointers in the layouts above;
 * q, k_pages, v_pages and out must be 16-byte aligned, the int32/fp32
 * arrays 4-byte aligned.  The device must be the one the plan was created
 * on.  Reads every input, writes only `out` and the plan's workspace. */
attn_status_t attn_paged_forward(attn_plan_t plan, const void* q, const uint8_t* k_pages,
                                 const uint8_t* v_pages, const float* kv_scales,
                                 const int32_t* block_table, const int32_t* ctx_lens,
                                 const int32_t* q_lens, void* out, hipStream_t stream);

/* Free the workspace and the plan.  The caller must first make sure no
 * forward using the plan is still running (synchronise its stream).
 * A null plan is accepted and ignored. */
attn_status_t attn_plan_destroy(attn_plan_t plan);

/* Fill *info with the plan's choices. */
attn_status_t attn_plan_get_info(attn_plan_t plan, attn_plan_info_t* info);

/* Measurement hook.  With both events non-null, every later forward on this
 * plan launches its attention kernel (and every attn_kv_append its append
 * kernel) with `attention_start` and `attention_stop` attached to the
 * kernel's own dispatch (hipExtLaunchKernel),
 * so hipEventElapsedTime gives that kernel's duration alone (the merge kernel
 * that may follow is not included).  Both null turns it off; exactly one null
 * is ATTN_ERR_INVALID_ARGUMENT.  The events stay owned by the caller and must
 * outlive their use; forwards under stream capture should not set them. */
attn_status_t attn_plan_set_kernel_events(attn_plan_t plan, hipEvent_t attention_start,
                                          hipEvent_t attention_stop);

/* Measurement hook, as attn_plan_set_kernel_events for the log-sum-exp merge
 * kernel a forward launches after the attention kernel when keys were split.
 * A forward that launches no merge records both events at the same point of
 * the stream (zero duration). */
attn_status_t attn_plan_set_merge_events(attn_plan_t plan, hipEvent_t merge_start, hipEvent_t merge_stop);

/* Measurement hook.  With `rows` non-null, every later forward on this plan
 * has each wave of its attention kernel record a timeline in its own row of
 * ATTN_TIMELINE_WORDS uint64 words of `rows` (device memory, 8-byte
 * aligned): row = workgroup * waves_per_group + wave, num_rows at least
 * grid_size * waves_per_group (attn_plan_get_info), else
 * ATTN_ERR_INVALID_ARGUMENT.  Word i < ATTN_TIMELINE_WORDS - 1 is the i-th
 * event, (t << 4) | type, t the GPU's constant-rate real-time counter
 * (wallclock_khz ticks per millisecond): type 1 the wave's start, 6 the
 * sequence lengths read and summed, 2 its chunk range known, then per
 * piece of a segment 3 its start, 4 each chunk
 * step (each group of chunks in the packed decode), 5 its end; events past
 * the row's first ATTN_TIMELINE_WORDS - 1 words are dropped.  The last word
 * is (t << 4) | 7 at the wave's end.  Words nothing writes keep their
 * contents: zero the rows before the forward.  Null turns it off.  The
 * forwards then run copies of the attention kernels built with the
 * recording (the others contain none of it), for E4M3 KV with bf16 q and
 * out only: other plans get ATTN_ERR_UNSUPPORTED.  The buffer stays owned
 * by the caller and must outlive its use. */
#define ATTN_TIMELINE_WORDS 64
attn_status_t attn_plan_set_timeline(attn_plan_t plan, uint64_t* rows, size_t num_rows);

/* ---- allocation-free forward ----
 * For callers that cannot allocate device memory: code under HIP graph
 * capture that must not call hipMalloc, tight serving loops, harnesses that
 * forbid allocation.  It computes exactly what attn_paged_forward computes
 * for a plan made from *desc (the same choices, kernels and result), but
 * takes the descriptor instead of a plan and keeps the split partials in a
 * library-owned device array of attn_static_scratch_bytes() bytes (32 MiB),
 * one per GPU, held until the process ends; it calls no hipMalloc or
 * hipFree.  The array's device address is looked up on the first call on
 * each device.
 *   desc, q .. out, stream: as attn_plan_create and attn_paged_forward (the
 *   current device is the one used).
 * Errors: as those two; ATTN_ERR_UNSUPPORTED when the workspace a plan for
 * *desc needs (attn_plan_info_t.workspace_bytes) exceeds the array, e.g. the
 * 8 x 512-token prefill chunk of 32 query / 8 kv heads (~100 MB).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (two streams, or two host threads) race and give wrong
 * results; calls on one stream are ordered and safe.  Nothing in the array
 * needs to start at zero (each forward writes what it reads). */
attn_status_t attn_paged_forward_static(const attn_plan_desc_t* desc, const void* q, const uint8_t* k_pages,
                                        const uint8_t* v_pages, const float* kv_scales, const int32_t* block_table,
                                        const int32_t* ctx_lens, const int32_t* q_lens, void* out,
                                        hipStream_t stream);

/* Size in bytes of the per-GPU array attn_paged_forward_static uses. */
size_t attn_static_scratch_bytes(void);

/* ---- the step before the attention: appending new tokens' K/V ----------
 * Follows the same passages as the attention (memory section: fixed-size
 * blocks of a preallocated pool; quantisation section: FP8 with per-group
 * scale factors; GB10 article: the paged FP8 KV cache that decode, MTP
 * verification and prefill append to).
 *
 * For each sequence b the Q_b rows k_new[r_b + i], v_new[r_b + i] (i < Q_b,
 * r_b = Q_0 + ... + Q_{b-1}) become keys L_b - Q_b + i, stored through
 * block_table[b] (so after the call L_b keys are cached, as the forward
 * expects).  For every (page, kv head) the append touches, separately for K
 * and V:
 *   value(slot) = decoded byte * old scale     for the L_b - Q_b cached keys
 *               = the new row's value           for the new keys
 *   scale       = fp32(max |value| over the page's keys < L_b) / 448,
 *                 1 if that maximum is 0
 *   byte(slot)  = nearest E4M3 code to fp32(value / scale), ties to even,
 *                 magnitudes above 448 saturated, sign kept
 * for every slot holding a key < L_b (cached keys are encoded again, and
 * keep their bytes exactly when the scale does not change); slots >= L_b and
 * pages the append does not touch keep their bytes.  The divisions and the
 * product are IEEE fp32, so the bytes and scales are exactly determined.
 *
 *   k_new, v_new  [sum Q_b][Hkv][D], new_dtype BF16 or F32, 16-byte aligned,
 *                 finite values
 *   k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens: as for the
 *                 forward (ctx_lens counts the appended tokens); k_pages and
 *                 v_pages 16-byte aligned, the int32/fp32 arrays 4-byte aligned.
 * Preconditions beyond the forward's: block_table[b][j] in [0, P) for the
 * pages j = (L_b - Q_b)/16 .. (L_b - 1)/16; no two sequences touch the same
 * page (each is written by one wave).  Asynchronous on `stream`; allocates
 * nothing; reads and writes only the pools and scales of the touched pages.
 * The plan supplies the shape (B, Hkv, D, P, max_pages_per_seq, max_q_len);
 * its kernel events, when set, are attached to this kernel's dispatch too. */
attn_status_t attn_kv_append(attn_plan_t plan, const void* k_new, const void* v_new, attn_dtype_t new_dtype,
                             uint8_t* k_pages, uint8_t* v_pages, float* kv_scales,
                             const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens,
                             hipStream_t stream);

/* ---- the step after MTP verification: greedy acceptance of the drafts ----
 * The GB10 article serves with multi-token prediction, K = 4 drafts, under
 * deterministic decoding.  For sequence b and position i <= K (row
 * r = b (K+1) + i of the target model's logits):
 *   target_tokens[r] = the lowest index v holding the largest logits[r][v]
 *                      (+0 and -0 are equal; logits finite)
 *   num_accepted[b]  = the largest n <= K with draft_tokens[b][j] ==
 *                      target_tokens[b (K+1) + j] for every j < n
 * (the tokens emitted are then target_tokens[b (K+1) + 0 .. n]).
 *   logits         [B][K+1][vocab] BF16 or F32, 16-byte aligned; vocab a
 *                  multiple of 8, at most 2^31 - 1
 *   draft_tokens   int32 [B][K]; target_tokens int32 [B][K+1];
 *   num_accepted   int32 [B]
 *   workspace      device memory of attn_mtp_accept_workspace_size() bytes,
 *                  8-byte aligned, owned by the caller (not kept)
 *   kernel_start, kernel_stop  measurement hook: when both are non-null they
 *                  are attached to the dispatch of the argmax kernel (the
 *                  one that reads the logits); null for normal use.
 * B (K+1) <= 65535.  Asynchronous on `stream`; allocates nothing.  Errors as
 * elsewhere: bad arguments return before any launch. */
size_t attn_mtp_accept_workspace_size(int32_t num_seqs, int32_t num_drafts, int32_t vocab);
attn_status_t attn_mtp_accept(const void* logits, attn_dtype_t logits_dtype, const int32_t* draft_tokens,
                              int32_t num_seqs, int32_t num_drafts, int32_t vocab, int32_t* target_tokens,
                              int32_t* num_accepted, void* workspace, size_t workspace_bytes,
                              hipEvent_t kernel_start, hipEvent_t kernel_stop, hipStream_t stream);

/* Static, never-null text for a status code. */
const char* attn_status_string(attn_status_t status);

/* The hipError_t (as int) of the last ATTN_ERR_HIP returned on this thread. */
int attn_last_hip_error(void);

/* ---- checking hooks: they run the same device address and FP8 decode code
 * as the attention kernels, so the gathered bytes can be compared bit for bit
 * with the oracle's gather. ---- */

/* For every sequence b < B, kv head h, token t < max_ctx_len:
 *   k_out[b][h][t][:], v_out[b][h][t][:]  the token's D K/V bytes (0 for t >= L_b)
 *   scale_out[0|1][b][h][t]               its K/V page scale (0 for t >= L_b)
 *   page_out[b][t]                        its physical page (-1 for t >= L_b)
 * Output buffers are caller-owned device memory of exactly those shapes. */
attn_status_t attn_debug_gather(attn_plan_t plan, const uint8_t* k_pages, const uint8_t* v_pages,
                                const float* kv_scales, const int32_t* block_table,
                                const int32_t* ctx_lens, uint8_t* k_out, uint8_t* v_out,
                                float* scale_out, int32_t* page_out, hipStream_t stream);

/* out[i] = the value of E4M3 byte in[i] as the attention kernels decode it
 * (FP8 -> bf16, widened exactly to fp32).  n >= 0; n == 0 enqueues nothing. */
attn_status_t attn_debug_decode_fp8(const uint8_t* in, float* out, int64_t n, hipStream_t stream);

/* out[i] = the value of INT8 byte in[i] (two's complement) as the attention
 * kernels widen it for ATTN_KV_INT8 pools (byte -> bf16, widened exactly to
 * fp32; the page scale is not applied).  in: n bytes, out: n floats, both
 * device memory, out 4-byte aligned.  n >= 0; n == 0 enqueues nothing;
 * n < 0 or a null pointer -> ATTN_ERR_INVALID_ARGUMENT. */
attn_status_t attn_debug_decode_int8(const uint8_t* in, float* out, int64_t n, hipStream_t stream);

/* out[2i + j] = the value of code j (bits 4j..4j+3, two's complement) of
 * byte in[i] as the attention kernels widen it for ATTN_KV_INT4 pools (the
 * page scale is not applied).  in: n bytes, out: 2n floats, both device
 * memory, out 4-byte aligned.  n >= 0; n == 0 enqueues nothing; n < 0 or a
 * null pointer -> ATTN_ERR_INVALID_ARGUMENT. */
attn_status_t attn_debug_decode_int4(const uint8_t* in, float* out, int64_t n, hipStream_t stream);

/* out[i] = the E4M3 byte of fp32 in[i] as the append kernel encodes it
 * (nearest code, ties to even, magnitudes above 448 saturated, sign kept;
 * finite inputs).  n >= 0; n == 0 enqueues nothing. */
attn_status_t attn_debug_encode_fp8(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

/* ---- measurement hook: the streaming-read ceiling ----
 * The HBM fraction of the attention kernels is reported against the MI355X
 * peak and against what this kernel reaches for the same access pattern: it
 * reads num_chunks chunks of chunk_bytes contiguous bytes, chunk i starting at
 * pool + chunk_ids[i] * chunk_bytes (a paged KV cache reads every (page, kv
 * head) as one such chunk, at a random place of the pool), with 16-byte
 * loads, `waves` waves each streaming an equal contiguous share of the list,
 * and writes one XOR word per lane to sink (waves * 64 uint32, so the loads
 * cannot be dropped).  No other arithmetic.
 *   access      0: the 64 lanes of a wave read 1 KB of whole 128-byte lines
 *               per instruction (the pattern of this library's page
 *               layouts); 1 (chunk_bytes >= 2048): each 2 KB is 16 rows of
 *               128 bytes, lane (q, r) (q = lane / 16, r = lane % 16) reads
 *               bytes 32 q + 16 i of row r in instruction i = 0, 1 -- half
 *               of 16 lines per instruction, the pattern of a [16 slots][128]
 *               byte layout read as 32 values of d per lane
 *   pool        device memory of pool_bytes (>= chunk_bytes), 16-byte aligned;
 *               ids outside [0, pool_bytes / chunk_bytes) are clamped into it
 *   chunk_ids   int32 [num_chunks], device memory
 *   chunk_bytes a power of two in [1024, 2^24]
 *   waves       1 .. 2^20
 *   kernel_start, kernel_stop  when both non-null, attached to the kernel's
 *               own dispatch (its duration alone); null otherwise.
 * Asynchronous on `stream`; allocates nothing.  Not part of the attention
 * path. */
attn_status_t attn_calib_stream_read(const uint8_t* pool, int64_t pool_bytes, const int32_t* chunk_ids,
                                     int64_t num_chunks, int32_t chunk_bytes, int32_t waves, int32_t access,
                                     uint32_t* sink, hipEvent_t kernel_start, hipEvent_t kernel_stop,
                                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
