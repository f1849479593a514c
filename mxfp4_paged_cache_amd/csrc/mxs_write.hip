// MXFP4 index-K writer (gfx950): bf16 keys [N, 128] quantized into their
// page slots (ATOM #2770, "Summary" and the write-path commit: the index key
// is quantized straight into its pool page slot; the conversion rule is not
// on the pages, this library follows the OCP Microscaling v1.0 conversion for
// FP4 E2M1 elements with an E8M0 scale per 32 elements):
//   e = floor(log2(amax)) - 2 per 32-element block, stored as byte e + 127
//   clipped to [1, 254]; each element is the e2m1 value nearest to x / 2^e,
//   ties to the even code, saturated at 6, sign kept.
// An fp8 cache (the format the MXFP4 one replaces, aiter #7061, "Summary")
// gets each element as the nearest e4m3 value (ties to even, saturated at
// +-448, unit scale), the rounding the query takes.
#include "mxs_device.h"

namespace mxs {
namespace {
using namespace dev;

// The element conversion is v_cvt_scalef32_pk_fp4_f32: two floats x0, x1 to
// the e2m1 codes of x0 / s and x1 / s (nearest, ties to the even code,
// saturated at 6, sign kept; x0 in the low nibble) in one byte of the
// destination. Measured on gfx950 against the rule above for values from
// -10 s to 10 s in steps of s / 8, the midpoints, signed zero and s from
// 2^-100 to 2^100: identical codes.

// Four tokens per step: lanes 16 s .. 16 s + 15 hold token 4 j + s, lane l
// of a token holds elements 8 l .. 8 l + 7 (one 16-byte load, one 4-byte
// store), and the 4 lanes 4 b .. 4 b + 3 one 32-element block (the block
// maximum takes two lane exchanges). A wave takes kWriteSteps steps at once,
// all loads first, so that enough bytes are in flight to cover the latency.
constexpr int kWriteSteps = 4;
// The cache bytes are stored non-temporally (they are not read back soon):
// 2^20 keys took 59 us against 71.5 us with ordinary stores on one MI355X.
// The keys themselves are read with ordinary loads (non-temporal loads as
// well measured slower than either alone).

template <int KDT>
__global__ void __launch_bounds__(kThreads) k_write(WArgs a) {
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4, l = lane & 15;
  const int64_t w0 = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const int64_t quads = (a.n + 3) / 4;
  // page size 64 or 128 (checked on the host): slot -> (page, offset) by shift and mask
  const int psh = a.P == 128 ? 7 : 6;
  for (int64_t w = w0; w * kWriteSteps < quads; w += nw) {
    int64_t slot[kWriteSteps], page[kWriteSteps];
    bool ok[kWriteSteps];
    uint4 raw[kWriteSteps];
#pragma unroll
    for (int u = 0; u < kWriteSteps; ++u) {
      const int64_t t = 4 * (w * kWriteSteps + u) + sub;
      const bool tok = t < a.n;
      slot[u] = tok ? a.slots[t] : -1;
      page[u] = slot[u] >= 0 ? slot[u] >> psh : -1;
      ok[u] = tok && slot[u] >= 0 && page[u] < a.num_pages;   // slots outside the pool are skipped
      // 8 bf16 elements (16 bytes); a skipped token reads row 0, which exists
      raw[u] = *reinterpret_cast<const uint4*>(a.k + (ok[u] ? t : 0) * a.k_row_stride + 8 * l);
    }
#pragma unroll
    for (int u = 0; u < kWriteSteps; ++u) {
      const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
      if constexpr (KDT == MXS_K_E4M3) {
        // fp8 cache: elements 8 l .. 8 l + 7 as e4m3 bytes, in element order
        const uint2 v = {(uint32_t)bf16x4_to_e4m3(w4[0], w4[1]), (uint32_t)bf16x4_to_e4m3(w4[2], w4[3])};
        if (ok[u]) {
          const int64_t off = slot[u] & (a.P - 1);
          typedef uint32_t u2 __attribute__((ext_vector_type(2)));
          __builtin_nontemporal_store(u2{v.x, v.y},
                                      reinterpret_cast<u2*>(a.kd + page[u] * a.kd_page_stride + off * 128 + 8 * l));
        }
        continue;
      }
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w4[i] << 16);
        x[2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      int ex = 0;
      (void)frexpf(amax, &ex);                                   // amax = m 2^ex, m in [0.5, 1)
      const int byte = amax > 0.0f ? min(254, max(1, ex - 1 - 2 + 127)) : 1;
      const int e = byte - 127;
      const float sc = __uint_as_float((uint32_t)(e + 127) << 23);   // 2^e, e in [-126, 127]
      uint32_t packed = 0;
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, x[0], x[1], sc, 0);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, x[2], x[3], sc, 1);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, x[4], x[5], sc, 2);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, x[6], x[7], sc, 3);
      if (ok[u]) {
        const int64_t off = slot[u] & (a.P - 1);
        __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t*>(a.kd + page[u] * a.kd_page_stride + off * 64 + 4 * l));
        if ((l & 3) == 0)
          __builtin_nontemporal_store((uint8_t)byte, a.ks + page[u] * a.ks_page_stride + off * 4 + (l >> 2));
      }
    }
  }
}

}  // namespace

hipError_t launch_write(int64_t grid, const WArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<WArgs*>(&a)};
  const void* fn = a.kdt == MXS_K_E4M3 ? reinterpret_cast<const void*>(&k_write<MXS_K_E4M3>)
                                       : reinterpret_cast<const void*>(&k_write<MXS_K_MXFP4>);
  return hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(kThreads), args, 0, stream);
}

}  // namespace mxs
