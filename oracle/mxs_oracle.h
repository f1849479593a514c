/*
 * mxs_oracle.h -- plain, slow CPU oracle for paged MXFP4 index scoring.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product path (the
 * HIP library under mxfp4_paged_cache_amd/) shares no code, header, table or
 * constant with it, and never calls it.
 *
 * What it computes (sources are the three pages this project follows):
 *   - MXFP4 element: e2m1 code times 2^(e8m0 byte - 127), one e8m0 byte per
 *     32 elements (aiter #7061, "Format"; ATOM #2770, "Summary").
 *   - Page of P tokens: data view [page][token][64 B], scale view
 *     [page][token][4 B], each with its own byte page stride (aiter #7061,
 *     "Format"; aiter #5518, "Summary").
 *   - fp8 index cache (the format the MXFP4 one replaces; aiter #7061,
 *     "Summary": 128 B per token): data view [page][token][128 B] of e4m3
 *     values, unit scale, no scale view.
 *   - Query: bf16 rounded to e4m3 (round to nearest even, saturating at 448,
 *     unit scale), or e4m3 bytes used as stored (aiter #7061, "Kernels";
 *     ATOM #2770, the write-path commit on the unit-scale saturating e4m3 q).
 *   - Mask: a query row sees tokens t < limit; prefill limit is
 *     min(seq_len, prefix_len + i + 1) for the request's i-th row, decode limit
 *     is seq_len (aiter #7061, "Kernels" and "Changed op tests").
 *   - logit = RN_fp32(sm_scale * exact dot), -inf outside the live window;
 *     block score = max over a page's live tokens (aiter #7061, "Format").
 * All arithmetic is exact until the single final rounding to fp32.
 */
#ifndef MXS_ORACLE_H
#define MXS_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

#define MXO_Q_BF16 1
#define MXO_Q_E4M3 2
#define MXO_K_MXFP4 0
#define MXO_K_E4M3 1
#define MXO_MODE_PREFILL 0
#define MXO_MODE_DECODE 1

/* Element decoders (exact in double). */
double mxo_e2m1_value(int code);   /* code 0..15, sign in bit 3 */
double mxo_e8m0_value(int byte);   /* 2^(byte-127); byte 255 -> NaN */
double mxo_e4m3_value(int byte);   /* OCP e4m3fn: bias 7, 0x7F/0xFF NaN */
/* bf16 bit pattern -> e4m3fn byte, round to nearest even, satfinite, NaN kept. */
int mxo_bf16_to_e4m3(int bf16_bits);

/* RN_fp32(sm_scale * sum_k S[k] * 2^(s[k]-127)), computed exactly then rounded
 * once. S[k] must be integer multiples of 2^-10 with |S[k]| < 2^17 (true for
 * 32-element block sums of e4m3 x e2m1 products). Returns NaN for byte 255. */
float mxo_round_scaled_sum(const double S[4], const int s[4], float sm_scale);

/* RN_fp32(sm_scale * sum_k S[k] * 2^ex[k]) for n <= 8 terms, computed exactly
 * then rounded once. Each S[k] * 2^frac_bits must be an integer below 2^62 in
 * magnitude (NaN is returned otherwise). */
float mxo_round_scaled_terms(const double* S, const int* ex, int n, int frac_bits, float sm_scale);

typedef struct mxo_args {
  int mode;                         /* MXO_MODE_PREFILL or MXO_MODE_DECODE */
  int q_dtype;                      /* MXO_Q_BF16 (uint16 bits) or MXO_Q_E4M3 (bytes) */
  const void* q;                    /* prefill: [T, H, 128]; decode: [B, H, 128] */
  int64_t q_row_stride, q_head_stride;   /* elements */
  int num_heads;
  const uint8_t* k_data; int64_t data_page_stride;    /* bytes; token stride 64 (MXFP4) or 128 (e4m3) */
  const uint8_t* k_scale; int64_t scale_page_stride;  /* bytes; MXFP4 only (NULL for e4m3) */
  int page_size;                    /* tokens per page */
  int64_t num_pages;                /* bound check on block-table entries */
  const int32_t* block_table; int64_t bt_row_stride; int bt_width;
  const int32_t* cu_seqlens_q;      /* [B+1], prefill only */
  const int32_t* seq_lens;          /* [B] */
  const int32_t* prefix_lens;       /* [B], prefill only */
  int batch;
  int max_seq_len;                  /* output window: logits width; NB = ceil(max_seq_len / P) */
  float sm_scale;
  const int32_t* rows;              /* optional subset of query rows (NULL = all rows) */
  int num_rows;                     /* rows in the subset (ignored when rows == NULL) */
  int num_threads;                  /* 0 = OpenMP default */
  int k_dtype;                      /* MXO_K_MXFP4 (e2m1 + e8m0 views) or MXO_K_E4M3 (128 e4m3 bytes per token) */
} mxo_args;

/* Score the selected rows. Outputs are dense and row-major over the selected
 * rows: logits [R, H, max_seq_len], blocks [R, H, NB], mags [R, H, max_seq_len]
 * (mags = sum over the 128 elements of |Q_hat * K|, without sm_scale, 0 for
 * dead tokens). Any output may be NULL. Returns 0, or a negative code:
 * -1 bad argument, -2 block-table entry of a live page out of range. */
int mxo_score(const mxo_args* a, float* logits, float* blocks, double* mags);

/* mxo_score plus block_mags [R, H, NB]: for each (row, head, page) the largest
 * mags value among the page's live tokens (0 when the page has none). That is
 * the M of a block score: a block score is the maximum of its page's logits,
 * so an error of at most eps * M_t on every logit t moves it by at most
 * eps * max_t M_t. Any output may be NULL. */
int mxo_score_ex(const mxo_args* a, float* logits, float* blocks, double* mags, double* block_mags);

/* Rows a selection would hold when rows == NULL. */
int mxo_total_rows(const mxo_args* a);

#ifdef __cplusplus
}
#endif
#endif
