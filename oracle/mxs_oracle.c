/*
 * mxs_oracle.c -- plain CPU oracle for paged MXFP4 index scoring.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by tests/, by the smoke check and by the
 * benchmark's CPU-baseline leg, never by the product library. It shares no
 * code with the GPU path. Every step follows the pages' definition directly:
 *
 *   K(p, j, e) = e2m1(code of element e of token j) * 2^(scale byte - 127),
 *                element 2m in the low nibble of data byte m, scale byte k
 *                covering elements 32k..32k+31
 *                (aiter #7061, "Format": e2m1 data plus one e8m0 scale per
 *                 32 elements; data view [pages, P, 64], scale view [pages, P, 4])
 *   Q_hat      = e4m3(Q): bf16 rounded to nearest even, saturating, unit
 *                scale; e4m3 input used as stored
 *                (aiter #7061, "Kernels"; ATOM #2770, write-path commit on
 *                 the unit-scale saturating e4m3 q)
 *   logit      = RN_fp32(sm_scale * sum_e Q_hat[e] * K[e]), the sum exact,
 *                -inf for tokens outside the row's live window
 *   block      = max over the page's live tokens of the logit, -inf if none
 *                (aiter #7061, "Format": max over live tokens of the dot)
 *
 * The dot is computed exactly: every product Q_hat * e2m1 is a multiple of
 * 2^-10 below 2^12, so each 32-element block sum S_k is exact in double. The
 * four block sums are then scaled by their e8m0 factors and by sm_scale and
 * summed in a 384-bit integer, and the total is rounded once to fp32.
 *
 * The fp8 index cache that the MXFP4 one replaces (aiter #7061, "Summary"
 * and "Kernels": 128 B of e4m3 per token against 68 B, 16 KB per 128-token
 * page) is read as K(p, j, e) = e4m3(byte e of token j), unit scale; the
 * same query, mask, logit and block rules apply.
 */
#include "mxs_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------ elements */

double mxo_e2m1_value(int code) {
  /* OCP e2m1 magnitudes for the 3 low bits; bit 3 is the sign. */
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double v = mag[code & 7];
  return (code & 8) ? -v : v;
}

double mxo_e8m0_value(int byte) {
  if (byte == 255) return NAN;
  return ldexp(1.0, byte - 127);
}

double mxo_e4m3_value(int byte) {
  int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);        /* subnormal: m/8 * 2^-6 */
  else
    v = ldexp(8.0 + m, e - 10);      /* normal: (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

int mxo_bf16_to_e4m3(int bf16_bits) {
  uint32_t u = (uint32_t)(bf16_bits & 0xFFFF) << 16;
  float f;
  double a;
  int sign = (bf16_bits & 0x8000) ? 0x80 : 0;
  memcpy(&f, &u, 4);
  if (isnan(f)) return sign | 0x7F;
  a = fabs((double)f);
  if (a >= 448.0) return sign | 0x7E;           /* saturate finite, also +-inf */
  if (a < ldexp(1.0, -6)) {
    /* subnormal range, spacing 2^-9; nearbyint rounds ties to even.
       A result of 8 is the smallest normal 2^-6, whose code is also 8. */
    return sign | (int)nearbyint(a * 512.0);
  } else {
    int ex, E;
    double m;
    frexp(a, &ex);                               /* a = f * 2^ex, f in [0.5, 1) */
    E = ex - 1;                                  /* a in [2^E, 2^(E+1)), E in [-6, 8] */
    m = nearbyint((ldexp(a, -E) - 1.0) * 8.0);   /* 3-bit mantissa, ties to even */
    if (m == 8.0) { m = 0.0; E += 1; }
    return sign | ((E + 7) << 3) | (int)m;
  }
}

/* ------------------------------------------------------------ exact rounding */

typedef struct { uint64_t w[6]; } big384;   /* two's complement */

static void big_add_shifted(big384* acc, int64_t v, int shift) {
  uint64_t t[6] = {0, 0, 0, 0, 0, 0};
  uint64_t mag = v < 0 ? (uint64_t)(-v) : (uint64_t)v;
  int li = shift / 64, bi = shift % 64, i;
  uint64_t carry;
  t[li] = mag << bi;
  if (bi && li + 1 < 6) t[li + 1] = mag >> (64 - bi);
  if (v < 0) {
    carry = 1;
    for (i = 0; i < 6; ++i) {
      uint64_t r = ~t[i] + carry;
      carry = (carry && r == 0) ? 1 : 0;
      t[i] = r;
    }
  }
  carry = 0;
  for (i = 0; i < 6; ++i) {
    uint64_t s = acc->w[i] + t[i];
    uint64_t c1 = s < acc->w[i];
    uint64_t s2 = s + carry;
    uint64_t c2 = s2 < s;
    acc->w[i] = s2;
    carry = c1 | c2;
  }
}

static int big_bit(const big384* a, int i) {
  if (i < 0 || i >= 384) return 0;
  return (int)((a->w[i / 64] >> (i % 64)) & 1u);
}

static int big_any_below(const big384* a, int i) {   /* any bit in [0, i) set */
  int li, k;
  if (i <= 0) return 0;
  li = i / 64;
  for (k = 0; k < li && k < 6; ++k)
    if (a->w[k]) return 1;
  if (li < 6 && (i % 64) && (a->w[li] & ((1ull << (i % 64)) - 1))) return 1;
  return 0;
}

static uint64_t big_bits(const big384* a, int lo, int n) {   /* n <= 32 */
  uint64_t r = 0;
  int k;
  for (k = 0; k < n; ++k) r |= (uint64_t)big_bit(a, lo + k) << k;
  return r;
}

float mxo_round_scaled_terms(const double* S, const int* ex, int n, int frac_bits, float sm_scale) {
  big384 acc;
  int k, sm_exp, base = 0, have = 0, h = -1, lsb, neg, i;
  int64_t sm_int;
  double frac;
  memset(&acc, 0, sizeof acc);
  if (n < 0 || n > 8) return NAN;
  for (k = 0; k < n; ++k) {
    double t = ldexp(S[k], frac_bits);
    if (isnan(S[k]) || !(fabs(t) < ldexp(1.0, 62)) || t != nearbyint(t)) return NAN;
  }
  if (!(sm_scale > 0.0f) || isinf(sm_scale)) return NAN;
  frac = frexp((double)sm_scale, &sm_exp);     /* sm_scale = frac * 2^sm_exp */
  sm_int = (int64_t)ldexp(frac, 24);           /* 24-bit integer significand */
  sm_exp -= 24;
  /* term k = N_k * sm_int * 2^(ex[k] - frac_bits + sm_exp), N_k = S[k] * 2^frac_bits */
  for (k = 0; k < n; ++k) {
    int e = ex[k] - frac_bits + sm_exp;
    if (S[k] == 0.0) continue;
    if (!have || e < base) base = e;
    have = 1;
  }
  if (!have) return 0.0f;
  for (k = 0; k < n; ++k) {
    int64_t N, hi, lo, sg;
    int sh;
    if (S[k] == 0.0) continue;
    N = (int64_t)ldexp(S[k], frac_bits);
    sg = N < 0 ? -1 : 1;
    hi = (sg * N) >> 31;                       /* |N| = hi * 2^31 + lo, both below 2^31 */
    lo = (sg * N) & 0x7FFFFFFF;
    sh = ex[k] - frac_bits + sm_exp - base;
    if (hi) big_add_shifted(&acc, sg * hi * sm_int, sh + 31);
    if (lo) big_add_shifted(&acc, sg * lo * sm_int, sh);
  }
  neg = (int)(acc.w[5] >> 63);
  if (neg) {   /* magnitude */
    uint64_t carry = 1;
    for (i = 0; i < 6; ++i) {
      uint64_t r = ~acc.w[i] + carry;
      carry = (carry && r == 0) ? 1 : 0;
      acc.w[i] = r;
    }
  }
  for (i = 5; i >= 0; --i)
    if (acc.w[i]) { h = i * 64 + 63 - __builtin_clzll(acc.w[i]); break; }
  if (h < 0) return 0.0f;
  /* value = mag * 2^base; keep 24 significant bits, or fewer below 2^-126 */
  lsb = h - 23;
  if (lsb < -149 - base) lsb = -149 - base;
  {
    double r;
    float f;
    if (lsb <= 0) {
      r = ldexp((double)big_bits(&acc, 0, 25), base);
    } else {
      uint64_t q = big_bits(&acc, lsb, 25);
      int rb = big_bit(&acc, lsb - 1);
      int sticky = big_any_below(&acc, lsb - 1);
      if (rb && (sticky || (q & 1))) q += 1;   /* round half to even */
      r = ldexp((double)q, lsb + base);
    }
    f = (float)r;   /* exact, or +inf past the fp32 range */
    return neg ? -f : f;
  }
}

float mxo_round_scaled_sum(const double S[4], const int s[4], float sm_scale) {
  int ex[4], k;
  for (k = 0; k < 4; ++k) {
    if (s[k] == 255 || isnan(S[k])) return NAN;
    if (ldexp(S[k], 10) != nearbyint(ldexp(S[k], 10))) abort();   /* block sums are multiples of 2^-10 */
    ex[k] = s[k] - 127;
  }
  return mxo_round_scaled_terms(S, ex, 4, 10, sm_scale);
}

/* ------------------------------------------------------------ scoring */

int mxo_total_rows(const mxo_args* a) {
  if (a->mode == MXO_MODE_DECODE) return a->batch;
  return a->cu_seqlens_q ? a->cu_seqlens_q[a->batch] : 0;
}

static int request_of_row(const mxo_args* a, int r) {
  int lo = 0, hi = a->batch - 1;
  if (a->mode == MXO_MODE_DECODE) return r;
  while (lo <= hi) {   /* cu_seqlens_q is non-decreasing: find b with cu[b] <= r < cu[b+1] */
    int mid = (lo + hi) / 2;
    if (a->cu_seqlens_q[mid + 1] <= r) lo = mid + 1;
    else if (a->cu_seqlens_q[mid] > r) hi = mid - 1;
    else return mid;
  }
  return -1;
}

static double q_hat(const mxo_args* a, int64_t row, int h, int e) {
  int64_t idx = row * a->q_row_stride + (int64_t)h * a->q_head_stride + e;
  if (a->q_dtype == MXO_Q_BF16)
    return mxo_e4m3_value(mxo_bf16_to_e4m3(((const uint16_t*)a->q)[idx]));
  return mxo_e4m3_value(((const uint8_t*)a->q)[idx]);
}

int mxo_score(const mxo_args* a, float* logits, float* blocks, double* mags) {
  return mxo_score_ex(a, logits, blocks, mags, NULL);
}

int mxo_score_ex(const mxo_args* a, float* logits, float* blocks, double* mags, double* block_mags) {
  int T, R, H, P, NB, W, err = 0;
  int64_t ri;
  if (!a || !a->q || !a->k_data || !a->block_table || !a->seq_lens) return -1;
  if (a->k_dtype != MXO_K_MXFP4 && a->k_dtype != MXO_K_E4M3) return -1;
  if (a->k_dtype == MXO_K_MXFP4 && !a->k_scale) return -1;
  if (a->mode == MXO_MODE_PREFILL && (!a->cu_seqlens_q || !a->prefix_lens)) return -1;
  if (a->q_dtype != MXO_Q_BF16 && a->q_dtype != MXO_Q_E4M3) return -1;
  if (a->num_heads <= 0 || a->page_size <= 0 || a->batch < 0 || a->max_seq_len < 0) return -1;
  T = mxo_total_rows(a);
  R = a->rows ? a->num_rows : T;
  H = a->num_heads;
  P = a->page_size;
  W = a->max_seq_len;
  NB = (W + P - 1) / P;
  if (a->rows)
    for (ri = 0; ri < R; ++ri)
      if (a->rows[ri] < 0 || a->rows[ri] >= T) return -1;
#ifdef _OPENMP
  if (a->num_threads > 0) omp_set_num_threads(a->num_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
#endif
  for (ri = 0; ri < R; ++ri) {
    int r = a->rows ? a->rows[ri] : (int)ri;
    int b = request_of_row(a, r);
    int limit, h, e, t;
    double* qv;
    if (b < 0) { err = -1; continue; }
    if (a->mode == MXO_MODE_DECODE) {
      limit = a->seq_lens[b];
    } else {
      int i = r - a->cu_seqlens_q[b];
      int64_t causal = (int64_t)a->prefix_lens[b] + i + 1;   /* integers: no int32 wrap */
      limit = a->seq_lens[b] < causal ? a->seq_lens[b] : (int)causal;
    }
    if (limit > W) limit = W;   /* the output window ends at max_seq_len */
    if (limit < 0) limit = 0;
    if (logits)
      for (h = 0; h < H; ++h)
        for (t = 0; t < W; ++t) logits[((int64_t)ri * H + h) * W + t] = -INFINITY;
    if (blocks)
      for (h = 0; h < H; ++h)
        for (t = 0; t < NB; ++t) blocks[((int64_t)ri * H + h) * NB + t] = -INFINITY;
    if (mags)
      for (h = 0; h < H; ++h)
        for (t = 0; t < W; ++t) mags[((int64_t)ri * H + h) * W + t] = 0.0;
    if (block_mags)
      for (h = 0; h < H; ++h)
        for (t = 0; t < NB; ++t) block_mags[((int64_t)ri * H + h) * NB + t] = 0.0;
    qv = (double*)malloc(sizeof(double) * (size_t)H * 128);
    for (h = 0; h < H; ++h)
      for (e = 0; e < 128; ++e) qv[h * 128 + e] = q_hat(a, r, h, e);
    for (t = 0; t < limit; ++t) {
      int j = t / P, slot = t % P, k;
      int64_t page;
      const uint8_t *dp, *sp;
      double kv[128];
      int sb[4];
      if (j >= a->bt_width) { err = -2; break; }
      page = a->block_table[(int64_t)b * a->bt_row_stride + j];
      if (page < 0 || page >= a->num_pages) { err = -2; break; }
      if (a->k_dtype == MXO_K_E4M3) {
        /* fp8 cache: 128 e4m3 bytes per token, unit scale. Products of two
           e4m3 values are multiples of 2^-18 below 2^18, so every block sum
           is exact in double; the four sums go to the exact rounding with
           exponent 0. */
        dp = a->k_data + page * a->data_page_stride + (int64_t)slot * 128;
        for (h = 0; h < H; ++h) {
          double S[4], mag = 0.0;
          int ex[4] = {0, 0, 0, 0};
          float logit;
          for (k = 0; k < 4; ++k) {
            double sum = 0.0;
            for (e = 32 * k; e < 32 * k + 32; ++e) {
              double p = qv[h * 128 + e] * mxo_e4m3_value(dp[e]);
              sum += p;
              mag += fabs(p);
            }
            S[k] = sum;
          }
          logit = mxo_round_scaled_terms(S, ex, 4, 18, a->sm_scale);
          if (logits) logits[((int64_t)ri * H + h) * W + t] = logit;
          if (mags) mags[((int64_t)ri * H + h) * W + t] = mag;
          if (block_mags) {
            double* mp = &block_mags[((int64_t)ri * H + h) * NB + j];
            if (mag > *mp) *mp = mag;
          }
          if (blocks) {
            float* bp = &blocks[((int64_t)ri * H + h) * NB + j];
            if (logit > *bp) *bp = logit;
          }
        }
        continue;
      }
      dp = a->k_data + page * a->data_page_stride + (int64_t)slot * 64;
      sp = a->k_scale + page * a->scale_page_stride + (int64_t)slot * 4;
      for (e = 0; e < 128; ++e) {
        int byte = dp[e / 2];
        int code = (e % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        kv[e] = mxo_e2m1_value(code);
      }
      for (k = 0; k < 4; ++k) sb[k] = sp[k];
      for (h = 0; h < H; ++h) {
        double S[4], mag = 0.0;
        float logit;
        for (k = 0; k < 4; ++k) {
          double sum = 0.0, msum = 0.0;
          for (e = 32 * k; e < 32 * k + 32; ++e) {
            sum += qv[h * 128 + e] * kv[e];
            msum += fabs(qv[h * 128 + e] * kv[e]);
          }
          S[k] = sum;
          mag += msum * mxo_e8m0_value(sb[k]);
        }
        logit = mxo_round_scaled_sum(S, sb, a->sm_scale);
        if (logits) logits[((int64_t)ri * H + h) * W + t] = logit;
        if (mags) mags[((int64_t)ri * H + h) * W + t] = mag;
        if (block_mags) {
          double* mp = &block_mags[((int64_t)ri * H + h) * NB + j];
          if (mag > *mp) *mp = mag;
        }
        if (blocks) {
          float* bp = &blocks[((int64_t)ri * H + h) * NB + j];
          if (logit > *bp) *bp = logit;
        }
      }
    }
    free(qv);
  }
  return err;
}
