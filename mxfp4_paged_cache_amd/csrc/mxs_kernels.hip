// gfx950 kernels of the paged MXFP4 index scorer.
//
// One instruction does the arithmetic: v_mfma_scale_f32_16x16x128_f8f6f4
// with the MXFP4 K tile as the fp4 operand, the e4m3 query tile as the fp8
// operand, the token's e8m0 byte as the fp4 operand's block scale and 127
// (x1) for the query (ATOM #2770, squashed pa_decode MXFP4 commit: one
// scaled MFMA per 16 tokens x 16 queries, K e8m0 byte as scaleA). Operand
// layout, measured on gfx950 with one-hot probes:
//   fp4 operand, lane (g = lane/16, i = lane%16): row/column i, elements
//     32g..32g+31, element 2m in the low nibble of byte m (16 bytes, 4 VGPRs);
//   fp8 operand, lane (g, i): row/column i, elements 16g..16g+15 in bytes
//     0..15 and 64+16g..64+16g+15 in bytes 16..31 (8 VGPRs), as the pages state;
//   block scale, lane (g, i): scales elements 32g..32g+31 of row/column i;
//   result C[16][16], lane (g, i) register v: C[4g + v][i].
// An MXFP4 token row is therefore fed to the MFMA exactly as it sits in the
// page: 16 contiguous bytes per lane, no dequantization (aiter #7061,
// "Kernels": the page stays MXFP4 and is the fp4 A operand).
//
// Query rounding: bf16 -> f32 (exact) -> clamp to +-448 -> v_cvt_pk_fp8_f32
// (round to nearest even, OCP e4m3 on gfx950). With the clamp this equals
// round-to-nearest-even with saturation for every finite bf16 input
// (checked exhaustively on gfx950); NaN stays NaN (aiter #7061, "Kernels").
//
// Scaling: logit = RN(RN(dot) * sm_scale); the block max is taken on the
// unscaled dots and scaled afterwards, which gives the same bits because
// sm_scale > 0 and rounding is monotone.
#include <limits.h>

#include "mxs_internal.h"

namespace mxs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

// Saturate to the largest finite e4m3 magnitude; NaN stays NaN. The NaN test
// is on the bits: this file is compiled without NaN semantics for float
// arithmetic (so the max folds need no quieting copies), and the only NaN
// that can reach the kernels is an out-of-contract query element.
__device__ __forceinline__ float clamp_e4m3(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const bool nan = (u & 0x7FFFFFFFu) > 0x7F800000u;
  return nan ? x : __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f);
}

// Four bf16 values (two dwords, element order low half first) -> four e4m3 bytes.
__device__ __forceinline__ int bf16x4_to_e4m3(uint32_t w0, uint32_t w1) {
  const float a = __builtin_bit_cast(float, w0 << 16);
  const float b = __builtin_bit_cast(float, w0 & 0xFFFF0000u);
  const float c = __builtin_bit_cast(float, w1 << 16);
  const float d = __builtin_bit_cast(float, w1 & 0xFFFF0000u);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a), clamp_e4m3(b), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(c), clamp_e4m3(d), r, true);
  return r;
}

template <int QDT>
__device__ __forceinline__ v8i load_q_slice(const uint8_t* p, int g);

// The fp8-operand slice of one 128-element query vector held by lane group g:
// elements 16g..16g+15 and 64+16g..64+16g+15. p == nullptr gives zeros
// (padding lanes beyond the last head or row).
template <int QDT>
__device__ __forceinline__ v8i load_q_tile(const uint8_t* p, int g) {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  if (p == nullptr) return r;
  return load_q_slice<QDT>(p, g);
}

template <int QDT>
__device__ __forceinline__ v8i load_q_slice(const uint8_t* p, int g) {
  v8i r;
  if constexpr (QDT == MXS_Q_E4M3) {
    const u4 lo = *reinterpret_cast<const u4*>(p + 16 * g);
    const u4 hi = *reinterpret_cast<const u4*>(p + 64 + 16 * g);
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  } else {
    const u4* lo = reinterpret_cast<const u4*>(p + 32 * g);         // bf16 elements 16g..
    const u4* hi = reinterpret_cast<const u4*>(p + 128 + 32 * g);   // bf16 elements 64+16g..
    const u4 a0 = lo[0], a1 = lo[1], b0 = hi[0], b1 = hi[1];
    r[0] = bf16x4_to_e4m3(a0[0], a0[1]); r[1] = bf16x4_to_e4m3(a0[2], a0[3]);
    r[2] = bf16x4_to_e4m3(a1[0], a1[1]); r[3] = bf16x4_to_e4m3(a1[2], a1[3]);
    r[4] = bf16x4_to_e4m3(b0[0], b0[1]); r[5] = bf16x4_to_e4m3(b0[2], b0[3]);
    r[6] = bf16x4_to_e4m3(b1[0], b1[1]); r[7] = bf16x4_to_e4m3(b1[2], b1[3]);
  }
  return r;
}

// C[token][query] for 16 tokens (fp4 A: 16 bytes per lane, block scale kscale)
// against 16 queries (fp8 B), fresh accumulator.
__device__ __forceinline__ v4f mma_kq(u4 k, v8i q, int kscale) {
  const v8i a = {(int)k[0], (int)k[1], (int)k[2], (int)k[3], 0, 0, 0, 0};
  const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, q, z, 4, 0, 0, kscale, 0, 127);
}

__device__ __forceinline__ float max4(v4f c) {
  return __builtin_fmaxf(__builtin_fmaxf(c[0], c[1]), __builtin_fmaxf(c[2], c[3]));
}

// running max m over the four values of one MFMA result
// (compiles to two v_max3_f32; the compiler inserts the MFMA-to-VALU wait states)
__device__ __forceinline__ float max_into(float m, v4f c) {
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(m, c[0]), c[1]), c[2]), c[3]);
}

// Max over the four lane groups (lanes i, i+16, i+32, i+48).
__device__ __forceinline__ float fold_groups(float m) {
  m = __builtin_fmaxf(m, __shfl_xor(m, 16));
  m = __builtin_fmaxf(m, __shfl_xor(m, 32));
  return m;
}

// Four consecutive logits starting at token t0 (a multiple of 4) of one
// (row, head) output row, clipped to the window W.
__device__ __forceinline__ void store_logits4(float* row, int t0, v4f v, int W, bool vec) {
  if (vec && t0 + 3 < W) {
    *reinterpret_cast<v4f*>(row + t0) = v;
  } else {
#pragma unroll
    for (int x = 0; x < 4; ++x)
      if (t0 + x < W) row[t0 + x] = v[x];
  }
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// ---------------------------------------------------------------------------
// Decode: one wave per (request, group of 64 heads, chunk of <= 64 pages).
// Each page is read by exactly one wave, so K goes straight from HBM into
// registers (staging it in LDS would buy nothing): per 16-token tile, lane
// (g, i) loads bytes 16g..16g+15 of token 16t+i (one 1 KB contiguous block
// per wave instruction) and e8m0 byte g of that token. Pages are double-
// buffered in registers: the loads of page j+2 are in flight while page j+1
// is scored. The chunk's page ids are read once into one VGPR (lane l holds
// the id of page j0 + l) and picked per page with readlane.
// ---------------------------------------------------------------------------
template <int P>
struct RegPage {
  u4 d[P / 16];
  int s[P / 16];
};

// One page into registers. dp/sp are the page's (uniform) bases; doff/soff the
// lane's byte offsets inside the page (data: 64 i + 16 g; scale: 4 i + g).
template <int P>
__device__ __forceinline__ void load_reg_page(RegPage<P>& kp, const uint8_t* dp, const uint8_t* sp, uint32_t doff,
                                              uint32_t soff) {
#pragma unroll
  for (int t = 0; t < P / 16; ++t) {
    kp.d[t] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(dp + doff + 1024u * t));
    kp.s[t] = __builtin_nontemporal_load(sp + soff + 64u * t);
  }
}

// Query tile for lane (g, i) of head h (a padding lane reads a valid head and
// zeroes the result, so the load itself is never divergent).
template <int QDT>
__device__ __forceinline__ v8i load_q_tile_masked(const uint8_t* p, int g, bool valid) {
  v8i r = load_q_slice<QDT>(p, g);
#pragma unroll
  for (int d = 0; d < 8; ++d) r[d] = valid ? r[d] : 0;
  return r;
}

// Score one register-resident page against the wave's four query tiles.
// MASK: the page holds the end of the live window (tokens >= lip are dead).
// The tile loop is software-pipelined by hand: the four MFMAs of tile t are
// issued before the results of tile t-1 are folded, and a scheduling fence
// after each step keeps only two tiles of results live.
template <int P, bool MASK, bool LG>
__device__ __forceinline__ void decode_page(const RegPage<P>& kp, const v8i (&qt)[4], int j, int lip, int g,
                                            const bool (&hv)[4], float* stage, int jrel, float* lg_row,
                                            const int64_t (&hoff)[4], const KArgs& a) {
  constexpr int TPP = P / 16;
  const float s = a.sm_scale;
  float m[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  v4f prev[4];
  const int lrel = lip - 4 * g;   // token 16 tp + 4 g + v is live iff 16 tp + v < lrel
#pragma unroll
  for (int t = 0; t <= TPP; ++t) {
    v4f cur[4];
    if (t < TPP) {
#pragma unroll
      for (int n = 0; n < 4; ++n) cur[n] = mma_kq(kp.d[t], qt[n], kp.s[t]);
    }
    if (t > 0) {
      const int tp = t - 1;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        v4f c = prev[n];
        if constexpr (MASK) {
#pragma unroll
          for (int v = 0; v < 4; ++v) c[v] = (16 * tp + v < lrel) ? c[v] : kNegInf;
        }
        m[n] = max_into(m[n], c);
        if constexpr (LG) {
          if (hv[n])
            store_logits4(lg_row + hoff[n] * a.lg_head_stride, j * P + 16 * tp + 4 * g, c * s, a.max_seq_len,
                          a.vec_lg);
        }
      }
    }
    if (t < TPP) {
#pragma unroll
      for (int n = 0; n < 4; ++n) prev[n] = cur[n];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const float r = fold_groups(m[n]);
    if (g == 0) stage[(16 * n + (threadIdx.x & 15)) * kDecodeStageStride + jrel] = r * s;
  }
}

template <int QDT, int P, bool LG>
__global__ void __launch_bounds__(kThreads, 2) k_decode(KArgs a) {
  constexpr int TPP = P / 16;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, i = lane & 15;
  // the wave index is uniform across the wave: keep everything derived from it scalar
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
  if (item >= a.items) return;
  const int hg = (int)(item % a.head_groups);
  const int64_t rest = item / a.head_groups;
  const int pc = (int)(rest % a.page_items);
  const int b = (int)(rest / a.page_items);

  const int limit = clampi(a.seq[b], 0, a.max_seq_len);
  const int live_pages = (limit + P - 1) / P;
  const int j0 = pc * a.pages_per_item;
  const int j1 = min(j0 + a.pages_per_item, a.NB);
  const int jl = min(j1, live_pages);                 // pages [j0, jl) are scored

  // the chunk's page ids first (lane l: page j0 + l), so their latency overlaps the query loads
  const int my_page = (j0 + lane < jl) ? a.bt[(int64_t)b * a.bt_stride + j0 + lane] : 0;
  v8i qt[4];
  bool hv[4];
  int64_t hoff[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int h = hg * kDecodeHeads + n * 16 + i;
    hv[n] = h < a.H;
    const int hc = hv[n] ? h : a.H - 1;
    hoff[n] = (int64_t)hc;
    qt[n] = load_q_tile_masked<QDT>(a.q + (int64_t)b * a.q_row_stride + (int64_t)hc * a.q_head_stride, g, hv[n]);
  }
  float* bs_row = a.bs + (int64_t)b * a.bs_row_stride;
  float* lg_row = LG ? a.lg + (int64_t)b * a.lg_row_stride : nullptr;
  // this wave's staging area for its block scores: [64 heads][pages of the chunk]
  __shared__ float stage_all[kWaves][kDecodeHeads * kDecodeStageStride];
  float* stage = stage_all[wave];

  if (j0 < jl) {
    const uint32_t doff = (uint32_t)(i * 64 + 16 * g);
    const uint32_t soff = (uint32_t)(i * 4 + g);
    auto load_page = [&](RegPage<P>& kp, int j) {
      const int jj = min(j, jl - 1);
      const int64_t page = __builtin_amdgcn_readlane(my_page, jj - j0);
      load_reg_page<P>(kp, a.kd + page * a.kd_page_stride, a.ks + page * a.ks_page_stride, doff, soff);
    };
    auto score = [&](const RegPage<P>& kp, int j) {
      const int lip = limit - j * P;                 // live tokens in this page
      if (lip >= P)
        decode_page<P, false, LG>(kp, qt, j, lip, g, hv, stage, j - j0, lg_row, hoff, a);
      else
        decode_page<P, true, LG>(kp, qt, j, lip, g, hv, stage, j - j0, lg_row, hoff, a);
    };
    RegPage<P> A, B;
    load_page(A, j0);
    load_page(B, j0 + 1);
    // the fences stop the scheduler from hoisting a refill above the scoring
    // of the buffer it overwrites (that would keep three pages live)
    for (int j = j0; j < jl; j += 2) {
      score(A, j);
      __builtin_amdgcn_sched_barrier(0);
      load_page(A, j + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (j + 1 < jl) score(B, j + 1);
      __builtin_amdgcn_sched_barrier(0);
      load_page(B, j + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // pages past the live window: -inf
  for (int j = max(j0, jl); j < j1; ++j) {
    if (g == 0)
#pragma unroll
      for (int n = 0; n < 4; ++n) stage[(16 * n + i) * kDecodeStageStride + (j - j0)] = kNegInf;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      if (hv[n]) {
        if constexpr (LG) {
          const v4f ninf = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
          for (int t = 0; t < TPP; ++t)
            store_logits4(lg_row + hoff[n] * a.lg_head_stride, j * P + 16 * t + 4 * g, ninf, a.max_seq_len, a.vec_lg);
        }
      }
    }
  }
  // Block scores leave LDS as one contiguous run of (j1 - j0) floats per head:
  // consecutive lanes write consecutive pages, so every store instruction
  // covers whole cache lines instead of 64 scattered 4-byte words.
  const int npg = j1 - j0;
  const int nh = min(kDecodeHeads, a.H - hg * kDecodeHeads);
  for (int idx = lane; idx < nh * npg; idx += 64) {
    const int h = idx / npg, p = idx - h * npg;
    bs_row[(int64_t)(hg * kDecodeHeads + h) * a.bs_head_stride + j0 + p] = stage[h * kDecodeStageStride + p];
  }
}

// ---------------------------------------------------------------------------
// Prefill (also the logits path for now): one workgroup per work item
// (request, block of 256 query slots, chunk of pages), looping over items
// with a grid stride. A query slot is (row, head); slot = row * H + head, so
// a 16-slot tile is 16 heads of one row when H is a multiple of 16. Each wave
// keeps 4 query tiles in registers for the whole item; every page is staged
// once per workgroup in LDS (double-buffered, 8.5 KB per buffer at P = 128)
// and read by all four waves. Block scores are staged in LDS for up to 32
// pages and leave as contiguous per-slot rows.
//
// Work items are ordered page chunk fastest. With a grid and a chunk count
// that are both multiples of 8, workgroup c only ever sees chunks c mod 8;
// workgroups are dispatched round-robin over the 8 XCDs, so each XCD reads
// one eighth of the pages and keeps them in its own L2.
// ---------------------------------------------------------------------------
template <int P>
struct PageStage {
  static constexpr int kDataChunks = P * 64 / 16 / kThreads;   // 16-byte chunks per thread
  u4 d[kDataChunks];
  uint32_t sc;
};

// LDS layout of a staged page: the data of 16-token tile t is stored as
// [lane group g][row i][16 bytes] at 1024 t + 256 g + 16 i, so the 16 lanes of
// a group read 256 contiguous bytes (no bank conflicts on ds_read_b128); the
// scales follow as [token][4 bytes] at P * 64. Thread tid fills LDS slot
// s = tid + 256 c (16 bytes, contiguous writes) with global bytes
// 16 g..16 g+15 of token 16 t + i, (t, g, i) = (s / 64, s / 16 % 4, s % 16):
// a wave still loads one contiguous 1 KB tile per instruction.
template <int P>
__device__ __forceinline__ void stage_load(PageStage<P>& st, const uint8_t* dp, const uint8_t* sp, int tid) {
#pragma unroll
  for (int c = 0; c < PageStage<P>::kDataChunks; ++c) {
    const int sl = tid + kThreads * c;
    const int off = ((sl >> 6) * 16 + (sl & 15)) * 64 + ((sl >> 4) & 3) * 16;
    st.d[c] = *reinterpret_cast<const u4*>(dp + off);
  }
  if (tid < P) st.sc = *reinterpret_cast<const uint32_t*>(sp + 4 * tid);
}

template <int P>
__device__ __forceinline__ void stage_store(const PageStage<P>& st, uint8_t* buf, int tid) {
#pragma unroll
  for (int c = 0; c < PageStage<P>::kDataChunks; ++c)
    *reinterpret_cast<u4*>(buf + 16 * (tid + kThreads * c)) = st.d[c];
  if (tid < P) *reinterpret_cast<uint32_t*>(buf + P * 64 + 4 * tid) = st.sc;
}

constexpr int kPrefillStagePages = 32;                      // pages per block-score flush
constexpr int kPrefillStageStride = kPrefillStagePages + 1; // LDS row pitch (odd: no bank conflicts)
constexpr int kPrefillSlots = kWaves * kPrefillTiles * 16;  // query slots per work item

// Score one LDS-resident page against this wave's query tiles; r[n] gets the
// (unscaled) max over the page's live tokens for slot (tile n, lane i).
// The 16-token tiles run in a real (not unrolled) loop, two per trip, so at
// most two tiles of MFMA results are live.
template <int P, bool MASK, bool LG>
__device__ __forceinline__ void prefill_page(const uint8_t* kb, const v8i (&qt)[kPrefillTiles],
                                             const int (&lrel)[kPrefillTiles], int j, int g, int i,
                                             float (&r)[kPrefillTiles], float* const (&lrow)[kPrefillTiles],
                                             const KArgs& a) {
  constexpr int TPP = P / 16;
  constexpr int NQ = kPrefillTiles;
  const uint8_t* kdl = kb + g * 256 + i * 16;     // this lane's 16 bytes of tile t: kdl + 1024 t
  const uint8_t* ksl = kb + P * 64 + i * 4 + g;   // this lane's scale byte of tile t: ksl + 64 t
  float m[NQ];
#pragma unroll
  for (int n = 0; n < NQ; ++n) m[n] = kNegInf;
  auto mma = [&](u4 k, int sc, v4f (&c)[NQ]) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) c[n] = mma_kq(k, qt[n], sc);
  };
  auto fold = [&](int t, const v4f (&cc)[NQ]) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      v4f c = cc[n];
      if constexpr (MASK) {
#pragma unroll
        for (int v = 0; v < 4; ++v) c[v] = (16 * t + v < lrel[n]) ? c[v] : kNegInf;
      }
      m[n] = max_into(m[n], c);
      if constexpr (LG) {
        if (lrow[n]) store_logits4(lrow[n], j * P + 16 * t + 4 * g, c * a.sm_scale, a.max_seq_len, a.vec_lg);
      }
    }
  };
  // two tiles per trip, no MFMA result carried across trips; the next pair of
  // K tiles is read from LDS while this pair is multiplied and folded
  u4 k0 = *reinterpret_cast<const u4*>(kdl);
  int s0 = ksl[0];
  u4 k1 = *reinterpret_cast<const u4*>(kdl + 1024);
  int s1 = ksl[64];
#pragma unroll 1
  for (int t = 0; t < TPP; t += 2) {
    v4f cA[NQ], cB[NQ];
    mma(k0, s0, cA);
    mma(k1, s1, cB);
    if (t + 2 < TPP) {
      k0 = *reinterpret_cast<const u4*>(kdl + 1024 * (t + 2));
      s0 = ksl[64 * (t + 2)];
      k1 = *reinterpret_cast<const u4*>(kdl + 1024 * (t + 3));
      s1 = ksl[64 * (t + 3)];
    }
    fold(t, cA);
    fold(t + 1, cB);
  }
#pragma unroll
  for (int n = 0; n < NQ; ++n) r[n] = fold_groups(m[n]);
}

template <int QDT, int P, bool WANT_BS, bool WANT_LG>
__global__ void __launch_bounds__(kThreads, 2) k_prefill(KArgs a) {
  constexpr int NQ = kPrefillTiles;
  constexpr int PB = P * 68;   // bytes of one staged page
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2 * PB];
  __shared__ float stage[WANT_BS ? kPrefillSlots * kPrefillStageStride : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i = lane & 15;
  const float s = a.sm_scale;
  const v4f ninf = {kNegInf, kNegInf, kNegInf, kNegInf};

  for (int64_t item = blockIdx.x; item < a.items; item += gridDim.x) {
    const int pc = (int)(item % a.page_items);
    const int64_t rest = item / a.page_items;
    const int sb = (int)(rest % a.slot_items);
    const int b = (int)(rest / a.slot_items);
    const int row0 = a.cu[b];
    const int qlen = a.cu[b + 1] - row0;
    const int64_t nslots = (int64_t)qlen * a.H;
    const int64_t sbeg = (int64_t)sb * kPrefillSlots;
    if (sbeg >= nslots) continue;   // uniform over the workgroup
    const int seq = a.seq[b], pre = a.prefix[b];
    const int64_t slast = min(sbeg + (int64_t)kPrefillSlots, nslots) - 1;
    const int item_lim = clampi(min(seq, pre + (int)(slast / a.H) + 1), 0, a.max_seq_len);

    // this lane's query slots
    v8i qt[NQ];
    int lim[NQ];
    float* lrow[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const int64_t sl = sbeg + (int64_t)(wave * NQ + n) * 16 + i;
      const bool valid = sl < nslots;
      const int64_t slc = valid ? sl : nslots - 1;
      const int r = (int)(slc / a.H);
      const int h = (int)(slc % a.H);
      const int64_t grow = (int64_t)row0 + r;
      lim[n] = valid ? clampi(min(seq, pre + r + 1), 0, a.max_seq_len) : 0;
      qt[n] = load_q_tile_masked<QDT>(a.q + grow * a.q_row_stride + (int64_t)h * a.q_head_stride, g, valid);
      lrow[n] = (WANT_LG && valid) ? a.lg + grow * a.lg_row_stride + (int64_t)h * a.lg_head_stride : nullptr;
    }
    // smallest limit among this wave's slots: the limit of its first slot
    const int64_t wfirst = sbeg + (int64_t)wave * NQ * 16;
    const int wave_min_lim = wfirst < nslots ? clampi(min(seq, pre + (int)(wfirst / a.H) + 1), 0, a.max_seq_len) : 0;

    const int j0 = pc * a.pages_per_item;
    const int j1 = min(j0 + a.pages_per_item, a.NB);
    const int jl = min(j1, (item_lim + P - 1) / P);   // pages [j0, jl) hold live tokens
    const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;

    if (j0 < jl) {
      PageStage<P> st;
      const int64_t page = btrow[j0];
      stage_load<P>(st, a.kd + page * a.kd_page_stride, a.ks + page * a.ks_page_stride, tid);
      stage_store<P>(st, kbuf, tid);
    }
    __syncthreads();
    int jbase = j0;
    for (int j = j0; j < j1; ++j) {
      float r[NQ];
      if (j < jl) {
        const bool more = j + 1 < jl;
        PageStage<P> nx;
        if (more) {
          const int64_t page = btrow[j + 1];
          stage_load<P>(nx, a.kd + page * a.kd_page_stride, a.ks + page * a.ks_page_stride, tid);
        }
        const uint8_t* kb = kbuf + ((j - j0) & 1) * PB;
        int lrel[NQ];
#pragma unroll
        for (int n = 0; n < NQ; ++n) lrel[n] = lim[n] - j * P - 4 * g;
        if ((j + 1) * P > wave_min_lim)
          prefill_page<P, true, WANT_LG>(kb, qt, lrel, j, g, i, r, lrow, a);
        else
          prefill_page<P, false, WANT_LG>(kb, qt, lrel, j, g, i, r, lrow, a);
        if (more) stage_store<P>(nx, kbuf + ((j + 1 - j0) & 1) * PB, tid);
      } else {
#pragma unroll
        for (int n = 0; n < NQ; ++n) r[n] = kNegInf;
        if constexpr (WANT_LG) {
#pragma unroll
          for (int n = 0; n < NQ; ++n)
            if (lrow[n])
#pragma unroll
              for (int t = 0; t < P / 16; ++t) store_logits4(lrow[n], j * P + 16 * t + 4 * g, ninf, a.max_seq_len, a.vec_lg);
        }
      }
      if constexpr (WANT_BS) {
        if (g == 0) {
#pragma unroll
          for (int n = 0; n < NQ; ++n) stage[((wave * NQ + n) * 16 + i) * kPrefillStageStride + (j - jbase)] = r[n] * s;
        }
      }
      __syncthreads();
      if constexpr (WANT_BS) {
        if (j - jbase == kPrefillStagePages - 1 || j == j1 - 1) {
          // flush pages [jbase, j]: 8 threads per slot row, 4 pages per thread,
          // so each group of 8 threads writes one contiguous run of the row
          const int npg = j - jbase + 1;
          const int nvalid = (int)min((int64_t)kPrefillSlots, nslots - sbeg);
          const int part = tid & 7;
          const bool vec = a.vec_bs && (jbase & 3) == 0 && 4 * part + 3 < npg;
          for (int sl = tid >> 3; sl < nvalid; sl += kThreads / 8) {
            if (4 * part >= npg) continue;
            const uint32_t slot = (uint32_t)(sbeg - (int64_t)(a.H) * (sbeg / a.H)) + (uint32_t)sl;  // slot - H * row(sbeg)
            const uint32_t dr = slot / (uint32_t)a.H;
            const int64_t grow = (int64_t)row0 + sbeg / a.H + dr;
            float* dst = a.bs + grow * a.bs_row_stride + (int64_t)(slot - dr * (uint32_t)a.H) * a.bs_head_stride + jbase +
                         4 * part;
            const float* src = stage + sl * kPrefillStageStride + 4 * part;
            if (vec) {
              const v4f v = {src[0], src[1], src[2], src[3]};
              *reinterpret_cast<v4f*>(dst) = v;
            } else {
              for (int x = 0; x < 4 && 4 * part + x < npg; ++x) dst[x] = src[x];
            }
          }
          __syncthreads();
          jbase = j + 1;
        }
      }
    }
  }
}

template <typename K>
int occ_of(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kernel), kThreads, 0) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

template <int QDT, int P>
hipError_t launch_qp(const mxs_plan& plan, const KArgs& a, hipStream_t stream) {
  const dim3 grid(plan.grid), block(kThreads);
  void* args[] = {const_cast<KArgs*>(&a)};
  const void* fn = nullptr;
  if (plan.kernel == KID_DECODE) {
    fn = a.lg ? reinterpret_cast<const void*>(&k_decode<QDT, P, true>) : reinterpret_cast<const void*>(&k_decode<QDT, P, false>);
  } else {
    const bool bs = a.bs != nullptr, lg = a.lg != nullptr;
    if (bs && lg) fn = reinterpret_cast<const void*>(&k_prefill<QDT, P, true, true>);
    else if (bs) fn = reinterpret_cast<const void*>(&k_prefill<QDT, P, true, false>);
    else fn = reinterpret_cast<const void*>(&k_prefill<QDT, P, false, true>);
  }
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

template <int QDT, int P>
int occupancy_qp(int32_t kernel) {
  if (kernel == KID_DECODE) return occ_of(&k_decode<QDT, P, false>);
  return occ_of(&k_prefill<QDT, P, true, false>);
}

}  // namespace

hipError_t launch(const mxs_plan& plan, const KArgs& a, hipStream_t stream) {
  if (plan.q_dtype == MXS_Q_BF16) {
    return plan.page_size == 128 ? launch_qp<MXS_Q_BF16, 128>(plan, a, stream) : launch_qp<MXS_Q_BF16, 64>(plan, a, stream);
  }
  return plan.page_size == 128 ? launch_qp<MXS_Q_E4M3, 128>(plan, a, stream) : launch_qp<MXS_Q_E4M3, 64>(plan, a, stream);
}

int occupancy(int32_t kernel, int32_t q_dtype, int32_t page_size) {
  if (q_dtype == MXS_Q_BF16)
    return page_size == 128 ? occupancy_qp<MXS_Q_BF16, 128>(kernel) : occupancy_qp<MXS_Q_BF16, 64>(kernel);
  return page_size == 128 ? occupancy_qp<MXS_Q_E4M3, 128>(kernel) : occupancy_qp<MXS_Q_E4M3, 64>(kernel);
}

}  // namespace mxs
