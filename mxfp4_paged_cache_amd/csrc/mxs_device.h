// Device helpers shared by the gfx950 scorer kernels (mxs_decode.hip,
// mxs_prefill.hip, mxs_logits.hip) and the writer. Not part of the public ABI.
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
#pragma once

#include <limits.h>

#include "mxs_internal.h"

namespace mxs {
namespace dev {

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

// Query tile for lane (g, i) of head h (a padding lane reads a valid head and
// zeroes the result, so the load itself is never divergent).
template <int QDT>
__device__ __forceinline__ v8i load_q_tile_masked(const uint8_t* p, int g, bool valid) {
  v8i r = load_q_slice<QDT>(p, g);
#pragma unroll
  for (int d = 0; d < 8; ++d) r[d] = valid ? r[d] : 0;
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
// (row, head) output row, clipped to the window W. Non-temporal stores: the
// logits stream out once, in whole 512-byte row segments, and bypassing the
// caches' allocation took the per-head logits of 1024 rows x 64 heads x 8192
// tokens from 442 us to 367 us on one MI355X.
__device__ __forceinline__ void store_logits4(float* row, int t0, v4f v, int W, bool vec) {
  if (vec && t0 + 3 < W) {
    __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(row + t0));
  } else {
#pragma unroll
    for (int x = 0; x < 4; ++x)
      if (t0 + x < W) __builtin_nontemporal_store(v[x], row + t0 + x);
  }
}

// ---------------------------------------------------------------------------
// K formats. MXFP4 (MXS_K_MXFP4): 64 data bytes + 4 e8m0 bytes per token, the
// fp4 operand as stored. fp8 (MXS_K_E4M3, the cache the MXFP4 one replaces,
// aiter #7061, "Summary"): 128 e4m3 bytes per token, fed as the fp8 operand
// in the query's element layout (bytes 16g..16g+15 and 64+16g..64+16g+15 of
// the token for lane group g), both scales 127 (x1).
// ---------------------------------------------------------------------------
template <int KDT>
struct KTile;
template <>
struct KTile<MXS_K_MXFP4> {
  u4 d;    // elements 32g..32g+31 of token i (16 bytes)
  int s;   // their e8m0 byte
};
template <>
struct KTile<MXS_K_E4M3> {
  u4 lo;   // elements 16g..16g+15
  u4 hi;   // elements 64+16g..64+16g+15
};

__device__ __forceinline__ v4f mma_tile(const KTile<MXS_K_MXFP4>& k, v8i q) { return mma_kq(k.d, q, k.s); }

__device__ __forceinline__ v4f mma_tile(const KTile<MXS_K_E4M3>& k, v8i q) {
  const v8i a = {(int)k.lo[0], (int)k.lo[1], (int)k.lo[2], (int)k.lo[3],
                 (int)k.hi[0], (int)k.hi[1], (int)k.hi[2], (int)k.hi[3]};
  const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, q, z, 0, 0, 0, 127, 0, 127);
}

// Bytes of one page staged in LDS.
template <int KDT, int P>
constexpr int kStagedPageBytes = KDT == MXS_K_E4M3 ? P * 128 : P * 68;

// LDS layout of a staged page. MXFP4: the data of 16-token tile t is stored
// as [lane group g][row i][16 bytes] at 1024 t + 256 g + 16 i, so the 16
// lanes of a group read 256 contiguous bytes (no bank conflicts on
// ds_read_b128); the scales follow as [token][4 bytes] at P * 64. fp8: tile t
// is [half h][g][row][16 bytes] at 2048 t + 1024 h + 256 g + 16 (i ^ (4 h + g)),
// half h holding bytes 64 h + 16 g .. + 15 of token 16 t + i. The XOR keeps
// the 16 lanes of a group on 16 distinct 16-byte slots of one 256-byte run
// when reading, and sends the 8 chunks of one token (written by 8 adjacent
// lanes) to 8 distinct banks when staging.
template <int KDT, int P>
__device__ __forceinline__ KTile<KDT> lds_tile(const uint8_t* kb, int g, int i, int t) {
  KTile<KDT> r;
  if constexpr (KDT == MXS_K_E4M3) {
    r.lo = *reinterpret_cast<const u4*>(kb + 2048 * t + 256 * g + 16 * (i ^ g));
    r.hi = *reinterpret_cast<const u4*>(kb + 2048 * t + 1024 + 256 * g + 16 * (i ^ (4 + g)));
  } else {
    r.d = *reinterpret_cast<const u4*>(kb + 1024 * t + 256 * g + 16 * i);
    r.s = kb[P * 64 + 64 * t + 4 * i + g];
  }
  return r;
}

// Byte offset of 16-byte chunk c (0..127: token c / 8 of the tile, chunk c % 8
// of its 128 bytes) of fp8 tile `tile` in the layout above.
__device__ __forceinline__ int fp8_chunk_slot(int tile, int c) {
  return tile * 2048 + ((c & 7) >> 2) * 1024 + (c & 3) * 256 + (((c >> 3) & 15) ^ (c & 7)) * 16;
}

// Order a wave's own LDS writes before its later LDS reads of other lanes'
// data (and reads before later writes): a wave's LDS operations complete in
// program order; the fences keep the compiler from moving them across.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One page of K staged through registers into LDS by a whole workgroup.
template <int KDT, int P>
struct PageStage {
  static constexpr int kDataChunks = P * (KDT == MXS_K_E4M3 ? 128 : 64) / 16 / kThreads;   // 16-byte chunks per thread
  u4 d[kDataChunks];
  uint32_t sc;
};

// MXFP4: thread tid fills LDS slot s = tid + 256 c (16 bytes, contiguous
// writes) with global bytes 16 g..16 g+15 of token 16 t + i, (t, g, i) =
// (s / 64, s / 16 % 4, s % 16): a wave still loads one contiguous 1 KB tile
// per instruction. fp8: thread tid loads global chunk s (bytes 16 s..16 s+15
// of the page: token s / 8, half (s / 4) % 2, group s % 4), so a wave loads
// 1 KB contiguously, and stores it at its place in the tile layout.
template <int KDT, int P>
__device__ __forceinline__ void stage_load(PageStage<KDT, P>& st, const uint8_t* dp, const uint8_t* sp, int tid) {
#pragma unroll
  for (int c = 0; c < PageStage<KDT, P>::kDataChunks; ++c) {
    const int sl = tid + kThreads * c;
    if constexpr (KDT == MXS_K_E4M3) {
      st.d[c] = *reinterpret_cast<const u4*>(dp + 16 * sl);
    } else {
      const int off = ((sl >> 6) * 16 + (sl & 15)) * 64 + ((sl >> 4) & 3) * 16;
      st.d[c] = *reinterpret_cast<const u4*>(dp + off);
    }
  }
  if constexpr (KDT == MXS_K_MXFP4) {
    if (tid < P) st.sc = *reinterpret_cast<const uint32_t*>(sp + 4 * tid);
  }
}

template <int KDT, int P>
__device__ __forceinline__ void stage_store(const PageStage<KDT, P>& st, uint8_t* buf, int tid) {
#pragma unroll
  for (int c = 0; c < PageStage<KDT, P>::kDataChunks; ++c) {
    const int sl = tid + kThreads * c;
    if constexpr (KDT == MXS_K_E4M3) {
      *reinterpret_cast<u4*>(buf + fp8_chunk_slot(sl >> 7, sl & 127)) = st.d[c];
    } else {
      *reinterpret_cast<u4*>(buf + 16 * sl) = st.d[c];
    }
  }
  if constexpr (KDT == MXS_K_MXFP4) {
    if (tid < P) *reinterpret_cast<uint32_t*>(buf + P * 64 + 4 * tid) = st.sc;
  }
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Tokens that query row i >= 0 (within its request) sees before the output
// window clips them: min(seq_len, prefix_len + i + 1) (aiter #7061,
// "Kernels": the causal limit of a prefill row). The sum is formed only when
// it is below seq_len, so no prefix_len, however large, wraps it.
__device__ __forceinline__ int causal_limit(int seq, int pre, int i) {
  return pre < seq - i ? pre + i + 1 : seq;
}

// Raw buffer resource over [base, base + bytes) (no stride, no swizzle).
// A buffer load at an offset at or past `bytes` returns zeros without a
// memory request, so bytes = 0 turns every load through the resource into a
// no-op that still issues and retires like any other load.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kNonTemporal = 2;   // cache-policy operand of a buffer load: nt (streamed once)
__device__ __forceinline__ u4 buffer_load16_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNonTemporal);
}
__device__ __forceinline__ uint32_t buffer_load4_nt(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kNonTemporal);
}
__device__ __forceinline__ int buffer_load1_nt(rsrc_t r, uint32_t off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, kNonTemporal);
}

}  // namespace dev
}  // namespace mxs
