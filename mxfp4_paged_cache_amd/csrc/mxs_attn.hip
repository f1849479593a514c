// Paged MXFP4 attention decode (gfx950): one query row per (row, kv head),
// K and V read as MXFP4 straight from their pages (ATOM #2770, "How it works"
// and the sparse attention commit: the selected pages' K and V feed a paged
// decode attention, one row per (token, kv head)).
//
// One workgroup per (row, kv head); its four waves take the row's 64-token
// units (a 128-token page is two) round-robin, each keeping an online softmax state (running max, sum and
// the unnormalised output) for the kv head's G <= 16 query heads, and merge
// the four states through LDS at the end; the output row is written once, as
// bf16. Per page and wave:
//   * Q.K: one v_mfma_scale_f32_16x16x128_f8f6f4 per 16-token tile, the
//     page's e2m1 tile as the fp4 operand with its e8m0 bytes as block scale
//     and the G query heads (e4m3) as the fp8 operand, as in the scorers;
//     result lane (g, i): tokens 4g..4g+3 of the tile, head i;
//   * softmax in exp2 units (the host folds log2(e) into the scale); the
//     probabilities are rounded to bf16, and the sum uses the rounded values
//     so that the weights of the output stay a convex combination;
//   * P.V: out^T[d][h] += V^T[d][t] P[t][h] with v_mfma_f32_16x16x32_bf16,
//     32 tokens per step. A 32-token step orders its tokens k = 8g + 2q + h
//     <-> token 16h + 4g + q (h = 0, 1: the first or second Q.K tile), so
//     lane (g, i) already holds its P operand (head i, k = 8g..8g+7), and
//     tokens x and x + 16 sit at adjacent k: a lane that loads both (two
//     contiguous 1 KB blocks per wave) writes their values for one head-dim
//     element as one 4-byte word. V is widened to bf16 exactly with
//     v_cvt_scalef32_pk_bf16_fp4 (e2m1 times a power of two is a bf16 value)
//     and transposed through the wave's LDS tile [d][k]: 80-byte rows (the 16
//     lanes of a ds_read_b128 hit distinct banks) and 64 more bytes before
//     each group of 32 rows (the four rows one store instruction writes land
//     in distinct banks). Dead tokens get a zero V scale and a -inf score, so
//     their bytes cannot reach the output.
#include "mxs_device.h"

namespace mxs {
namespace {
using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kVPitch = 40;                        // bf16 per row of the transposed V chunk
constexpr int kVTileBytes = 128 * kVPitch * 2 + 3 * 64;   // one 32-token chunk, [128 d][40] + group offsets
constexpr int kOPitch = 132;                       // floats per (wave, head) row of the merge area
constexpr int kAttnLds = kWaves * kVTileBytes;     // also holds the merge area (4 x 16 x 132 floats)
static_assert(kWaves * 16 * kOPitch * 4 <= kAttnLds, "merge area must fit in the V tiles");

// K and V of one 64-token unit in registers (tokens slot0..slot0+63 of a
// page). K tile t, lane (g, i): bytes 16g..16g+15 of token 16t+i and its e8m0
// byte g. V chunk c (32 tokens), lane L: tokens 32c + x and 32c + 16 + x
// (x = L / 4), bytes 16(L % 4)..+15 of each (head dim 32(L % 4)..+31) and
// their e8m0 byte L % 4.
constexpr int kUnit = 64;
struct AttnUnit {
  u4 kd[kUnit / 16];
  int ks[kUnit / 16];
  u4 va[kUnit / 32], vb[kUnit / 32];
  int vsa[kUnit / 32], vsb[kUnit / 32];
};

// Loads go through buffer resources over the unit's bytes; a unit past the
// row's context gets empty resources (its loads return zeros and read
// nothing), so every unit's loads issue unconditionally and the waits on one
// unit never cover the loads of the next (with the loads under a branch,
// each unit waited for the next one's loads as well).
__device__ __forceinline__ void load_attn_unit(AttnUnit& pg, const AArgs& a, int64_t page, int slot0, int hk,
                                               int lane, bool live) {
  const int g = lane >> 4, i = lane & 15;
  const rsrc_t kd = buffer_rsrc(a.kd + page * a.kd_page_stride + (int64_t)hk * a.kd_head_stride + slot0 * 64,
                                live ? kUnit * 64 : 0);
  const rsrc_t ks = buffer_rsrc(a.ks + page * a.ks_page_stride + (int64_t)hk * a.ks_head_stride + slot0 * 4,
                                live ? kUnit * 4 : 0);
  const rsrc_t vd = buffer_rsrc(a.vd + page * a.vd_page_stride + (int64_t)hk * a.vd_head_stride + slot0 * 64,
                                live ? kUnit * 64 : 0);
  const rsrc_t vs = buffer_rsrc(a.vs + page * a.vs_page_stride + (int64_t)hk * a.vs_head_stride + slot0 * 4,
                                live ? kUnit * 4 : 0);
#pragma unroll
  for (int t = 0; t < kUnit / 16; ++t) {
    pg.kd[t] = buffer_load16_nt(kd, (uint32_t)((16 * t + i) * 64 + 16 * g));
    pg.ks[t] = buffer_load1_nt(ks, (uint32_t)((16 * t + i) * 4 + g));
  }
  const int x = lane >> 2, pp = lane & 3;
#pragma unroll
  for (int c = 0; c < kUnit / 32; ++c) {
    const int tok = 32 * c + x;
    pg.va[c] = buffer_load16_nt(vd, (uint32_t)(tok * 64 + 16 * pp));
    pg.vb[c] = buffer_load16_nt(vd, (uint32_t)((tok + 16) * 64 + 16 * pp));
    pg.vsa[c] = buffer_load1_nt(vs, (uint32_t)(tok * 4 + pp));
    pg.vsb[c] = buffer_load1_nt(vs, (uint32_t)((tok + 16) * 4 + pp));
  }
}

// byte offset of element (d, k) of the transposed V tile
__device__ __forceinline__ int vt_at(int d, int k) { return d * (kVPitch * 2) + 64 * (d >> 5) + 2 * k; }

// The four bytes of src (8 e2m1 elements, element 2m in the low nibble of
// byte m) times scale, as four packed bf16 pairs (pair m: elements 2m, 2m+1).
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t src, float scale, uint32_t (&out)[4]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scale, 0));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scale, 1));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scale, 2));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scale, 3));
}

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Three workgroups per CU (the LDS allows three): measured 5% faster than
// two with the larger register budget.
template <int QDT, int P>
__global__ void __launch_bounds__(kThreads, 3) k_attn(AArgs a) {
  constexpr int TPP = kUnit / 16, CPP = kUnit / 32;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kAttnLds];
  __shared__ float mm[kWaves][16], ll[kWaves][16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i = lane & 15;
  const int r = (int)(blockIdx.x / (uint32_t)a.Hkv), hk = (int)(blockIdx.x % (uint32_t)a.Hkv);
  const int ctx = clampi(a.ctx[r], 0, a.max_context);
  const int nunits = (ctx + kUnit - 1) / kUnit;
  const float c2 = a.scale_log2e;

  // the kv head's query heads as the fp8 operand (columns past G are zero)
  const bool hv = i < a.G;
  const v8i qt = load_q_tile_masked<QDT>(
      a.q + (int64_t)r * a.q_row_stride + (int64_t)(hk * a.G + (hv ? i : a.G - 1)) * a.q_head_stride, g, hv);

  float m_run = kNegInf, l_run = 0.0f;
  v4f o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  uint8_t* vt = lds + wave * kVTileBytes;
  const int32_t* btrow = a.bt + (int64_t)r * a.bt_stride;

  auto process = [&](const AttnUnit& pg, int j) {
    // Q.K and mask
    v4f s[TPP];
#pragma unroll
    for (int t = 0; t < TPP; ++t) s[t] = mma_kq(pg.kd[t], qt, pg.ks[t]) * c2;
    const int lip = ctx - j * kUnit;   // live tokens of this unit
    if (lip < kUnit) {
#pragma unroll
      for (int t = 0; t < TPP; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) s[t][v] = (16 * t + 4 * g + v < lip) ? s[t][v] : kNegInf;
    }
    // online softmax: page maximum per head, rescale of the running state
    float mp = kNegInf;
#pragma unroll
    for (int t = 0; t < TPP; ++t) mp = max_into(mp, s[t]);
    mp = fold_groups(mp);
    const float m_new = __builtin_fmaxf(m_run, mp);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    uint32_t pb[TPP][4];
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < TPP; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pb[t][v] = bf16_bits(__builtin_amdgcn_exp2f(s[t][v] - m_new));
        psum += __builtin_bit_cast(float, pb[t][v] << 16);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] *= alpha;
    // P.V, 32 tokens per step
    const int x = lane >> 2, pp = lane & 3;
    const int ka = 8 * (x >> 2) + 2 * (x & 3);   // k of token x; token x + 16 is at ka + 1
#pragma unroll
    for (int c = 0; c < CPP; ++c) {
      const int tok = j * kUnit + 32 * c + x;
      const float sa = tok < ctx ? __builtin_bit_cast(float, (uint32_t)pg.vsa[c] << 23) : 0.0f;
      const float sb = tok + 16 < ctx ? __builtin_bit_cast(float, (uint32_t)pg.vsb[c] << 23) : 0.0f;
      wave_lds_sync();   // the previous step's reads of vt are done
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t ua[4], ub[4];
        fp4x8_to_bf16(pg.va[c][w], sa, ua);
        fp4x8_to_bf16(pg.vb[c][w], sb, ub);
#pragma unroll
        for (int bsel = 0; bsel < 4; ++bsel) {
          // head-dim elements d0, d0 + 1 of tokens x (k = ka) and x + 16 (k = ka + 1)
          const int d0 = 32 * pp + 8 * w + 2 * bsel;
          *reinterpret_cast<uint32_t*>(vt + vt_at(d0, ka)) = __builtin_amdgcn_perm(ub[bsel], ua[bsel], 0x05040100u);
          *reinterpret_cast<uint32_t*>(vt + vt_at(d0 + 1, ka)) = __builtin_amdgcn_perm(ub[bsel], ua[bsel], 0x07060302u);
        }
      }
      wave_lds_sync();
      // k = 8g + 2q + h: token 4g + q of tile 2c + h
      const u4 pw = {pb[2 * c][0] | (pb[2 * c + 1][0] << 16), pb[2 * c][1] | (pb[2 * c + 1][1] << 16),
                     pb[2 * c][2] | (pb[2 * c + 1][2] << 16), pb[2 * c][3] | (pb[2 * c + 1][3] << 16)};
      const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const u4 vw = *reinterpret_cast<const u4*>(vt + vt_at(16 * db + i, 8 * g));
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vw), pop, o[db], 0, 0, 0);
      }
    }
  };

  // units wave, wave + 4, ...: register double buffer, the next unit's loads
  // in flight while this one is processed
  {
    auto load = [&](AttnUnit& u, int j) {
      const bool live = j < nunits;
      const int t0 = (live ? j : 0) * kUnit;
      load_attn_unit(u, a, live ? btrow[t0 / P] : 0, t0 % P, hk, lane, live);
    };
    AttnUnit A, B;
    int j = wave;
    load(A, j);
    for (; j < nunits; j += 2 * kWaves) {
      load(B, j + kWaves);
      process(A, j);
      if (j + kWaves >= nunits) break;
      load(A, j + 2 * kWaves);
      process(B, j + kWaves);
    }
  }

  // merge the four waves' states
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();   // every wave is done with its V tile: the merge area reuses it
  float* ob = reinterpret_cast<float*>(lds);
  if (g == 0) {
    mm[wave][i] = m_run;
    ll[wave][i] = l_run;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db) *reinterpret_cast<v4f*>(ob + (wave * 16 + i) * kOPitch + 16 * db + 4 * g) = o[db];
  __syncthreads();
  const int d = tid & 127;
  for (int h = tid >> 7; h < a.G; h += 2) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = __builtin_fmaxf(M, mm[w][h]);
    float val = 0.0f;
    if (M != kNegInf) {
      float L = 0.0f, O = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(mm[w][h] - M);
        L += ll[w][h] * f;
        O += ob[(w * 16 + h) * kOPitch + d] * f;
      }
      val = O / L;
    }
    __builtin_nontemporal_store((uint16_t)bf16_bits(val),
                                a.out + (int64_t)r * a.out_row_stride + (int64_t)(hk * a.G + h) * a.out_head_stride + d);
  }
}

template <int QDT, int P>
hipError_t launch_qp(const AArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<AArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&k_attn<QDT, P>), dim3((uint32_t)a.R * (uint32_t)a.Hkv),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_attn(int32_t q_dtype, int32_t page_size, const AArgs& a, hipStream_t stream) {
  if (q_dtype == MXS_Q_BF16)
    return page_size == 128 ? launch_qp<MXS_Q_BF16, 128>(a, stream) : launch_qp<MXS_Q_BF16, 64>(a, stream);
  return page_size == 128 ? launch_qp<MXS_Q_E4M3, 128>(a, stream) : launch_qp<MXS_Q_E4M3, 64>(a, stream);
}

}  // namespace mxs
