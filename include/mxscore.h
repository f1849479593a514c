/*
 * mxscore.h -- C ABI of the MI355X (gfx950) paged MXFP4 index scorer.
 *
 * The library scores query rows against a paged MXFP4 index-K cache and
 * writes fp32 logits scaled by sm_scale per (row, head, token) and per-page
 * maxima ("block scores") per (row, head, page).
 *
 * Cache format (aiter #7061, "Format"): each token holds 128 elements as
 * e2m1 codes, two per byte with element 2m in the low nibble of byte m
 * (64 B), plus four e8m0 scale bytes, byte k scaling elements 32k..32k+31
 * (4 B). Element value = e2m1(code) * 2^(byte - 127). A page holds P = 64 or
 * 128 tokens. The caller picks the layout through two views, each with its
 * own byte page stride (aiter #7061, "Format"; aiter #5518, "Summary"):
 *     data  byte i of token j of page p: data  + p*data_page_stride  + j*64 + i
 *     scale byte k of token j of page p: scale + p*scale_page_stride + j*4  + k
 * Split tensors, a single-region page [P x 64 B data][P x 4 B scales] and a
 * shared multi-slot pool past 4 GiB are all expressed this way; page offsets
 * are computed in 64 bits.
 *
 * fp8 index cache (the format the MXFP4 one replaces; aiter #7061,
 * "Summary": 128 B of e4m3 per token against 68 B, and "Kernels": a
 * 16 KB buffer per 128-token page): k_dtype = MXS_K_E4M3 selects pages of
 * 128 e4m3 (OCP float8_e4m3fn) bytes per token with unit scale, element e
 * at byte e; the data view is the only view:
 *     data  byte e of token j of page p: data  + p*data_page_stride  + j*128 + e
 * Everything else (query, mask, scores, outputs) is the same for both.
 *
 * Query (aiter #7061, "Kernels"; ATOM #2770, write-path commit): 128
 * elements per (row, head), bf16 rounded in-kernel to e4m3 (nearest even,
 * saturating at +-448, unit scale), or e4m3 (OCP float8_e4m3fn) used as stored.
 *
 * Scores: logit(r, h, t) = RN_fp32(RN_fp32(dot) * sm_scale) for live tokens,
 * where dot is the scaled-MFMA dot of Q_hat and K (see the error note below);
 * -inf for dead tokens. block(r, h, j) = max over live tokens t of page j of
 * logit(r, h, t), -inf when the page has none (aiter #7061, "Format").
 * Live tokens of a prefill row i of request b: t < min(seq_len[b],
 * prefix_len[b] + i + 1, max_seq_len); of a decode row b: t < min(seq_len[b],
 * max_seq_len) (aiter #7061, "Kernels" and "Changed op tests").
 *
 * Arithmetic note: the dot uses gfx950's block-scaled fp4 x fp8 MFMA
 * (ATOM #2770, squashed pa_decode MXFP4 commit: one
 * v_mfma_scale_f32_16x16x128_f8f6f4 per 16 tokens x 16 queries, the K e8m0
 * byte as its block scale). Measured on gfx950: the instruction sums products
 * across groups of 8 adjacent elements exactly and rounds once, but within a
 * group keeps about 12 bits below the group's largest product. Results equal
 * RN_fp32 of the exact dot except under cancellation, with
 * |error| <= 2^-11 * sum_e |Q_hat[e] K[e]| in the worst measured case.
 * An fp8 cache runs the same instruction with both operands e4m3 and unit
 * scales.
 *
 * Outputs: every element of the window is written: logits [rows, heads,
 * max_seq_len] and block scores [rows, heads, ceil(max_seq_len / P)]; live
 * entries get scores, everything else -inf, so no pre-fill is needed
 * (aiter #5518, "Correctness": outputs poisoned between graph replays must
 * be fully rewritten). Rows of requests with no query rows do not exist.
 *
 * Ownership and execution: every pointer in these structs is a device
 * pointer owned by the caller. Calls validate all host-visible arguments
 * first and touch no memory when they fail. A successful call enqueues its
 * kernels on `stream` (a hipStream_t; NULL = the null stream), returns
 * without synchronizing, allocates no device memory, keeps no pointer, and
 * may be captured in a HIP graph. Device-side contract (not checked):
 * cu_seqlens_q non-decreasing with cu_seqlens_q[B] == total_rows, each
 * request's q_len <= max_query_len, block-table entries of live pages in
 * [0, num_pages), e8m0 bytes (MXFP4) of live tokens in [1, 254], no NaN
 * e4m3 byte (0x7F, 0xFF) in live tokens of an fp8 cache. Entries past a
 * request's live pages are never read (they may hold -1).
 *
 * Thread safety: calls may be made from several host threads; error text is
 * kept per thread.
 */
#ifndef MXSCORE_H
#define MXSCORE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define MXS_OK 0
#define MXS_EINVAL (-1)       /* null pointer, negative count, sm_scale not finite and > 0 */
#define MXS_EDTYPE (-2)       /* query dtype not bf16 / e4m3 (fp16 is refused), or unknown cache dtype */
#define MXS_ELAYOUT (-3)      /* stride, alignment, page size or table width rule broken */
#define MXS_EUNSUPPORTED (-4) /* current device is not gfx950, or no device */
#define MXS_EDEVICE (-5)      /* HIP runtime error while launching */

/* ---------------------------------------------------------------- dtypes / modes */
#define MXS_Q_BF16 1
#define MXS_Q_E4M3 2

#define MXS_K_MXFP4 0         /* cache: e2m1 data + e8m0 scales (68 B per token) */
#define MXS_K_E4M3 1          /* cache: e4m3 data, unit scale (128 B per token) */

#define MXS_MODE_PREFILL 1
#define MXS_MODE_DECODE 2
#define MXS_MODE_LOGITS 3

/* Paged MXFP4 cache views (see the layout above).
 * data: 16-byte aligned, data_page_stride a multiple of 16 and >= 64 * page_size
 * (MXS_K_E4M3: >= 128 * page_size).
 * scale: 4-byte aligned, scale_page_stride a multiple of 4 and >= 4 * page_size
 * (MXS_K_MXFP4 only; ignored for MXS_K_E4M3 and may be NULL). */
typedef struct mxs_kcache {
  const void* data;
  int64_t data_page_stride;    /* bytes */
  const void* scale;
  int64_t scale_page_stride;   /* bytes */
  int32_t page_size;           /* 64 or 128 */
  int32_t k_dtype;             /* MXS_K_MXFP4 (0) or MXS_K_E4M3 (1) */
  int64_t num_pages;           /* pages addressable through the view(s), >= 1 */
} mxs_kcache;

/* Query rows: element e of head h of row r at
 * ptr + (r * row_stride + h * head_stride + e) * elem_size; head_dim 128 contiguous.
 * ptr 16-byte aligned; row_stride and head_stride (elements, >= 0) times the
 * element size multiples of 16 bytes. Prefill/logits rows are the
 * concatenated query rows [total_rows]; decode rows are requests [batch]. */
typedef struct mxs_query {
  const void* ptr;
  int32_t dtype;               /* MXS_Q_BF16 or MXS_Q_E4M3 */
  int64_t row_stride;          /* elements */
  int64_t head_stride;         /* elements */
  int32_t num_heads;           /* >= 1 */
} mxs_query;

/* fp32 output [rows, heads, width], last axis contiguous:
 * element (r, h, x) at ptr + r * row_stride + h * head_stride + x (elements).
 * ptr 4-byte aligned; strides >= 0. A NULL ptr means "not requested". With
 * no rows or max_seq_len = 0 a scoring call writes nothing and is a no-op,
 * and a required output may then be NULL too (an empty tensor's pointer). */
typedef struct mxs_out {
  float* ptr;
  int64_t row_stride;
  int64_t head_stride;
} mxs_out;

/* Request metadata (aiter #7061, "Kernels": block_table, cu_seqlens_q,
 * seq_lens, prefix_lens, max_query_len, max_seq_len). Device int32 arrays,
 * contiguous. bt_row_stride in int32 elements (aiter #5518, "Summary"). */
typedef struct mxs_batch {
  const int32_t* block_table;  /* [batch, bt_row_stride] */
  int64_t bt_row_stride;       /* >= bt_width */
  int32_t bt_width;            /* >= ceil(max_seq_len / page_size) */
  const int32_t* cu_seqlens_q; /* [batch + 1]; prefill/logits only (ignored by decode) */
  const int32_t* seq_lens;     /* [batch] */
  const int32_t* prefix_lens;  /* [batch]; prefill/logits only (ignored by decode) */
  int32_t batch;               /* >= 0 */
  int32_t total_rows;          /* prefill/logits: cu_seqlens_q[batch]; decode: ignored */
  int32_t max_query_len;       /* prefill/logits: >= every request's q_len; decode: ignored */
  int32_t max_seq_len;         /* output window in tokens, 0 .. 2^31 - 256 */
} mxs_batch;

/* Launch plan: a pure function of host integers (mode, shapes, page size,
 * the device's CU count and the kernels' occupancy), so a captured graph
 * replays the same launch (aiter #5518, decode auto-CTA: host-known buckets,
 * no device-to-host sync). Plain old data; may be computed once and reused
 * for every call with the same shapes. */
typedef struct mxs_plan {
  int32_t mode;
  int32_t q_dtype;
  int32_t page_size;
  int32_t num_heads;
  int32_t batch;
  int32_t max_query_len;
  int32_t max_seq_len;
  int32_t want_logits;
  int32_t want_blocks;
  int32_t grid;                /* workgroups launched */
  int32_t block;               /* threads per workgroup */
  int32_t slots_per_item;      /* (row, head) query slots per work item */
  int32_t pages_per_item;      /* pages per work item */
  int32_t slot_items;          /* work items along the slot axis, per request */
  int32_t page_items;          /* work items along the page axis, per request */
  int32_t head_groups;         /* decode: groups of 64 heads */
  int64_t items;               /* total work items */
  int32_t kernel;              /* internal kernel id */
  int32_t k_dtype;             /* cache dtype the plan was made for */
  int32_t xcd_split;           /* logits kernel: 1 = each of the 8 XCDs takes a contiguous eighth of the
                                  work items (query slots split across XCDs), 0 = workgroups stride over all
                                  items (page chunks split across XCDs); 0 for the other kernels */
} mxs_plan;

/* Compute a plan. parallel_unit_num > 0 overrides the workgroup count
 * (aiter #5518: explicit parallel_unit_num remains an override); 0 = auto.
 * For MXS_MODE_DECODE, max_query_len is ignored (1). k_dtype is the cache's
 * (MXS_K_MXFP4 or MXS_K_E4M3). Returns MXS_OK or an error code; writes *plan
 * only on success. */
int mxs_plan_make(int32_t mode, int32_t q_dtype, int32_t k_dtype, int32_t page_size, int32_t num_heads, int32_t batch,
                  int32_t max_query_len, int32_t max_seq_len, int32_t want_logits, int32_t want_blocks,
                  int32_t parallel_unit_num, mxs_plan* plan);

/* The same planner as a pure function of its arguments: num_cus is the
 * device's compute-unit count and wg_per_cu the workgroups of the chosen
 * kernel resident per CU (mxs_plan_make reads both from the current device).
 * Identical arguments always give an identical plan. */
int mxs_plan_make_for(int32_t mode, int32_t q_dtype, int32_t k_dtype, int32_t page_size, int32_t num_heads, int32_t batch,
                      int32_t max_query_len, int32_t max_seq_len, int32_t want_logits, int32_t want_blocks,
                      int32_t parallel_unit_num, int32_t num_cus, int32_t wg_per_cu, mxs_plan* plan);

/* Prefill block scorer (aiter #7061, "Kernels": score_prefill; the MXFP4
 * index-cache prefill scorer). Rows are the request-concatenated query rows.
 * block_scores required ([total_rows, H, NB]); logits optional
 * ([total_rows, H, max_seq_len]). plan may be NULL (computed per call). */
int mxs_score_prefill(const mxs_query* q, const mxs_kcache* k, const mxs_batch* batch, float sm_scale,
                      const mxs_out* block_scores, const mxs_out* logits, const mxs_plan* plan, void* stream);

/* Decode block scorer (ATOM #2770, "How it works": the MXFP4 index decode
 * scorer over the two views). One query row per request: q rows are the
 * requests, limit = seq_len. block_scores required ([batch, H, NB]); logits
 * optional ([batch, H, max_seq_len]). */
int mxs_score_decode(const mxs_query* q, const mxs_kcache* k, const mxs_batch* batch, float sm_scale,
                     const mxs_out* block_scores, const mxs_out* logits, const mxs_plan* plan, void* stream);

/* Logits-first scorer (aiter #5518, "Summary": paged MXFP4 MQA logits with
 * ragged query lengths). Same arguments and masking as prefill, tiled for
 * coalesced logit writes; logits required, block_scores optional. */
int mxs_score_logits(const mxs_query* q, const mxs_kcache* k, const mxs_batch* batch, float sm_scale,
                     const mxs_out* logits, const mxs_out* block_scores, const mxs_plan* plan, void* stream);

/* MXFP4 index-K writer (ATOM #2770, "Summary" and the write-path commit:
 * the index key is quantized straight into its pool page slot; the pages give
 * no conversion rule, this library uses the OCP Microscaling v1.0 one for FP4
 * E2M1 with an E8M0 scale per 32 elements). Token t of k (bf16 [num_tokens,
 * 128], head_dim contiguous, row stride in elements, 16-byte aligned rows)
 * goes to slot slot_mapping[t] = page * page_size + offset (int64; -1, or a
 * page past cache->num_pages, skips the token): for each 32-element block,
 * e = floor(log2(amax)) - 2 is stored as the e8m0 byte e + 127 clipped to
 * [1, 254], and each element as the e2m1 code nearest to x / 2^e (ties to the
 * even code, saturated at 6, sign kept), element 2m in the low nibble of
 * data byte m. Writes 64 data bytes and 4 scale bytes per token into the
 * cache views and nothing else. For an fp8 cache (MXS_K_E4M3) each element
 * becomes the e4m3 byte nearest to it (ties to even, saturated at +-448,
 * unit scale: the query rounding above), 128 bytes per token in the data
 * view. Non-finite keys are outside the contract.
 * Two tokens with the same slot race. Asynchronous on stream; num_tokens = 0
 * is a no-op. Returns MXS_OK, MXS_EINVAL, MXS_ELAYOUT, MXS_EUNSUPPORTED or
 * MXS_EDEVICE. */
int mxs_write_pages(const void* k, int64_t k_row_stride, int64_t num_tokens, const int64_t* slot_mapping,
                    const mxs_kcache* cache, void* stream);

/* Top-k page selection over block scores (ATOM #2770, "How it works": the
 * selection follows the scorer, and the squashed sparse-attention commit: the
 * tail page is always selected; k, the tie rule and the result order are this
 * library's reading). For every (row, head) of block_scores [rows, H, NB]
 * (as written by the scoring calls: -inf for pages holding no visible
 * token), writes to pages [rows, H, k] (int32, device memory owned by the
 * caller):
 *   - the tail page, (limit - 1) / page_size, where limit is the row's
 *     visible token count (prefill: min(seq_len, prefix_len + i + 1) for the
 *     request's i-th row; decode: seq_len; both clipped to max_seq_len);
 *   - the other live pages (finite score) with the largest scores, ties to
 *     the lower page index, up to k pages in all;
 *   in ascending page order, then -1 for places left when fewer than k pages
 *   are live. NB = ceil(max_seq_len / page_size), at most 4096.
 * mode: MXS_MODE_DECODE (rows are requests; batch->seq_lens used) or
 * MXS_MODE_PREFILL / MXS_MODE_LOGITS (rows per cu_seqlens_q; seq_lens and
 * prefix_lens used). batch->block_table is not read and may be NULL; with
 * max_seq_len = 0 no score is read and block_scores may be NULL (every row
 * gets k times -1). Strides in elements. Same device contract and asynchrony
 * as the scoring calls; k = 0 or no rows is a no-op. Returns MXS_OK, MXS_EINVAL,
 * MXS_ELAYOUT, MXS_EUNSUPPORTED (NB > 4096 or not gfx950) or MXS_EDEVICE. */
int mxs_select_pages(int32_t mode, const mxs_batch* batch, int32_t num_heads, int32_t page_size,
                     const float* block_scores, int64_t bs_row_stride, int64_t bs_head_stride, int32_t k,
                     int32_t* pages, int64_t pages_row_stride, int64_t pages_head_stride, void* stream);

/* Check of the device-side contract that the scoring calls cannot verify
 * without a device-to-host copy (see "Device contract" above). Synchronous:
 * copies the request metadata (and, with check_scales, the scale bytes, or
 * for an fp8 cache the data bytes, of every live token) to host memory after the work already queued on stream,
 * and checks, for mode MXS_MODE_PREFILL / MXS_MODE_LOGITS:
 *   cu_seqlens_q[0] == 0, non-decreasing, cu_seqlens_q[batch] == total_rows,
 *   every request's q_len <= max_query_len, prefix_lens >= 0;
 * for every mode:
 *   0 <= seq_lens[b] <= max_seq_len;
 *   block-table entries of live pages (pages holding a token some row of the
 *   request sees) in [0, num_pages);
 *   with check_scales != 0: e8m0 bytes of live tokens in [1, 254] (MXFP4),
 *   or no NaN byte (0x7F, 0xFF) in live tokens (fp8 cache).
 * Returns MXS_OK, or MXS_EINVAL naming the first violation (mxs_last_error),
 * or MXS_EDEVICE if a copy fails. For tests and debugging: not on the hot
 * path and not capturable in a graph. Allocates host memory only. */
int mxs_check_metadata(int32_t mode, const mxs_kcache* k, const mxs_batch* batch, int32_t check_scales, void* stream);

/* ---------------------------------------------------------------- attention decode */

/* One MXFP4 tensor (K or V) of a paged cache with kv heads, in two views:
 *     data  byte e of token j, kv head hk, page p: data  + p*data_page_stride  + hk*data_head_stride  + j*64 + e
 *     scale byte k of token j, kv head hk, page p: scale + p*scale_page_stride + hk*scale_head_stride + j*4  + k
 * (the index cache's format per (page, kv head): element 2m in the low nibble
 * of data byte m, scale byte k covering elements 32k..32k+31). data 16-byte
 * aligned with strides multiples of 16; scale 4-byte aligned with strides
 * multiples of 4. A single-region page [P x 64 B data][P x 4 B scales] per
 * (page, kv head) is data = base, scale = base + 64 P with equal strides. */
typedef struct mxs_kvview {
  const void* data;
  int64_t data_page_stride;    /* bytes */
  int64_t data_head_stride;    /* bytes */
  const void* scale;
  int64_t scale_page_stride;   /* bytes */
  int64_t scale_head_stride;   /* bytes */
} mxs_kvview;

typedef struct mxs_kvcache {
  mxs_kvview k;
  mxs_kvview v;
  int32_t page_size;           /* 64 or 128 */
  int32_t num_kv_heads;        /* >= 1 */
  int64_t num_pages;           /* pages addressable through every view, >= 1 */
} mxs_kvcache;

/* Paged MXFP4 attention decode, one query row per row (ATOM #2770, "How it
 * works" and the sparse attention commit: the selected pages' K and V are
 * read as MXFP4 by a paged decode attention, one row per (token, kv head);
 * the K/V format as above). For row r and query head h (kv head
 * hk = h / G, G = q->num_heads / kv->num_kv_heads, 1 <= G <= 16) over the
 * row's live tokens t < min(context_lens[r], max_context) (max_context
 * 0 .. 2^31 - 256):
 *     s_t = scale * (Q_hat[r, h] . K[t]),  out[r, h] = sum_t softmax(s)_t V[t]
 * Q_hat is the query rounded as the scorers round it (bf16 -> e4m3, nearest
 * even, saturating, unit scale; e4m3 used as stored). Token t of row r is in
 * page block_table[r * bt_row_stride + t / P], slot t % P. Output: bf16
 * [num_rows, Hq, 128], element (r, h, d) at out + (r * out_row_stride +
 * h * out_head_stride + d) * 2 bytes (strides in elements, >= 0); a row with
 * no live token gets zeros. Arithmetic: Q.K by the block-scaled MFMA (as in
 * the scorers), softmax in fp32 (exp2), P rounded to bf16 and V widened to
 * bf16 exactly for a bf16 MFMA with fp32 accumulation, one bf16 rounding of
 * the normalized output. Device contract: block-table entries of live pages
 * in [0, num_pages), e8m0 bytes of live tokens in [1, 254]. One kernel
 * launch, no allocation, asynchronous on stream. Returns MXS_OK, MXS_EINVAL,
 * MXS_EDTYPE, MXS_ELAYOUT, MXS_EUNSUPPORTED or MXS_EDEVICE. */
int mxs_attn_decode(const mxs_query* q, const mxs_kvcache* kv, const int32_t* block_table, int64_t bt_row_stride,
                    int32_t bt_width, const int32_t* context_lens, int32_t num_rows, int32_t max_context, float scale,
                    void* out, int64_t out_row_stride, int64_t out_head_stride, void* stream);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* mxs_last_error(void);

/* Library version string. */
const char* mxs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXSCORE_H */
