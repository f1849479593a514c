// Top-k page selection over block scores (gfx950).
//
// For every (row, head) of a block-score tensor [rows, H, NB]: the tail page
// (the page holding the row's last visible token) and the k - 1 best other
// live pages (largest score, ties to the lower page index), written in
// ascending page order and padded with -1 (ATOM #2770, "How it works": the
// selection follows the scorer; the sparse-attention commit: the tail page is
// always selected; k and the tie rule are this library's reading).
#include "mxs_device.h"

namespace mxs {
namespace {
using namespace dev;

// One wave per (row, head); lane l holds the scores of pages 64 m + l, so
// every load instruction reads 256 contiguous bytes, and the lanes below l
// with a set ballot bit are exactly the lower pages of round m.
//
// Scores become order-preserving unsigned keys; pages without a visible token
// (-inf) get key 0 and the tail page the largest key, so it is always chosen.
// A bitwise search over the key finds T, the k-th largest key among the live
// pages (k clipped to their count); the result is every page with key > T and
// the lowest-indexed pages with key == T, emitted in page order.
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t ballot_count(bool p) { return __builtin_popcountll(__ballot(p)); }

template <int PER>
__global__ void __launch_bounds__(kThreads) k_select(SArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  for (int64_t item = wave; item < a.items; item += nw) {
    const int64_t r = item / a.H;
    const int h = (int)(item - r * a.H);
    // the row's visible tokens, as the scorer masks them
    int lim;
    if (a.decode) {
      lim = a.seq[r];
    } else {
      int lo = 0, hi = a.B - 1;   // request b with cu[b] <= r < cu[b + 1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu[mid] <= r) lo = mid; else hi = mid - 1;
      }
      lim = min(a.seq[lo], a.prefix[lo] + (int)(r - a.cu[lo]) + 1);
    }
    lim = clampi(lim, 0, a.max_seq_len);
    const int tail = lim > 0 ? (lim - 1) / a.P : -1;

    const float* srow = a.bs + r * a.bs_row_stride + (int64_t)h * a.bs_head_stride;
    uint32_t key[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int j = 64 * m + lane;
      const float s = j < a.NB ? srow[j] : kNegInf;
      key[m] = (s - s == 0.0f) ? (j == tail ? 0xFFFFFFFFu : order_key(s)) : 0u;   // finite test
    }
    uint32_t live = 0;
#pragma unroll
    for (int m = 0; m < PER; ++m) live += ballot_count(key[m] != 0u);
    const uint32_t keff = min((uint32_t)a.k, live);

    int32_t* orow = a.out + r * a.out_row_stride + (int64_t)h * a.out_head_stride;
    uint32_t written = 0;
    if (keff > 0) {
      uint32_t T = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        uint32_t cnt = 0;
#pragma unroll
        for (int m = 0; m < PER; ++m) cnt += ballot_count(key[m] >= cand);
        if (cnt >= keff) T = cand;
      }
      uint32_t gt = 0;
#pragma unroll
      for (int m = 0; m < PER; ++m) gt += ballot_count(key[m] > T);
      const uint32_t need_eq = keff - gt;
      uint32_t eq_seen = 0;
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        const bool eq = key[m] == T;
        const uint64_t beq = __ballot(eq);
        const uint32_t eq_rank = eq_seen + __builtin_amdgcn_mbcnt_hi((uint32_t)(beq >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)beq, 0u));
        const bool sel = key[m] > T || (eq && eq_rank < need_eq);
        const uint64_t bsel = __ballot(sel);
        const uint32_t pos = written + __builtin_amdgcn_mbcnt_hi((uint32_t)(bsel >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bsel, 0u));
        if (sel) orow[pos] = 64 * m + lane;
        written += __builtin_popcountll(bsel);
        eq_seen += __builtin_popcountll(beq);
      }
    }
    for (uint32_t p = written + lane; p < (uint32_t)a.k; p += 64) orow[p] = -1;
  }
}

}  // namespace

hipError_t launch_select(int per, int64_t grid, const SArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<SArgs*>(&a)};
  const void* fn = per <= 4    ? reinterpret_cast<const void*>(&k_select<4>)
                   : per <= 8  ? reinterpret_cast<const void*>(&k_select<8>)
                   : per <= 16 ? reinterpret_cast<const void*>(&k_select<16>)
                   : per <= 32 ? reinterpret_cast<const void*>(&k_select<32>)
                               : reinterpret_cast<const void*>(&k_select<64>);
  return hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(kThreads), args, 0, stream);
}

}  // namespace mxs
