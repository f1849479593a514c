// Top-k page selection over block scores (gfx950).
//
// For every (row, head) of a block-score tensor [rows, H, NB]: the tail page
// (the page holding the row's last visible token) and the k - 1 best other
// live pages (largest score, ties to the lower page index), written in
// ascending page order and padded with -1 (ATOM #2770, "How it works": the
// selection follows the scorer; the sparse-attention commit: the tail page is
// always selected; k and the tie rule are this library's reading).
#include <type_traits>

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
// The result is every page whose key exceeds T, the k-th largest key (k
// clipped to the live pages), and the lowest-indexed pages whose key equals
// T, emitted in page order. T comes from a radix search (6 bits per round):
//   * pruning: if each of n lanes holds j keys >= some x, then n j keys are
//     >= x; with x the smallest such j-th lane key (j = 2 or 1) and k <= n j,
//     T >= x, so only keys >= x are candidates; they are compacted in page
//     order into LDS and searched with as few registers per lane as they need;
//   * every candidate but the tail lies in [x, K] (K the largest non-tail
//     key), so T shares the leading bits x and K have in common and only the
//     bits below them are searched.
// Negative scores map to 0 - bits, which sends -0.0 to the key of +0.0 (the
// two compare equal, so they tie and the lower page wins) and keeps every
// other negative below it in order; a live key is never 0.
__device__ __forceinline__ uint32_t order_key_bits(uint32_t b) {
  return (b & 0x80000000u) ? 0u - b : (b | 0x80000000u);
}
__device__ __forceinline__ uint32_t order_key(float s) { return order_key_bits(__float_as_uint(s)); }

__device__ __forceinline__ uint32_t ballot_count(bool p) { return __builtin_popcountll(__ballot(p)); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Wave-wide min / max as a uniform value, with DPP row shifts (lane i takes
// lane i - n of its 16-lane row; lanes with no source keep the identity),
// then the row-15 and row-31 broadcasts: lane 63 ends with the result.
template <bool MIN>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x) {
  constexpr int id = MIN ? -1 : 0;   // identity: 0xFFFFFFFF for min, 0 for max
  auto op = [](uint32_t a, uint32_t b) { return MIN ? min(a, b) : max(a, b); };
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x111, 0xF, 0xF, false));   // row_shr:1
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x112, 0xF, 0xF, false));   // row_shr:2
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x114, 0xF, 0xF, false));   // row_shr:4
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x118, 0xF, 0xF, false));   // row_shr:8
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x142, 0xA, 0xF, false));   // row_bcast:15
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) { return wave_reduce<true>(x); }
__device__ __forceinline__ uint32_t wave_max(uint32_t x) { return wave_reduce<false>(x); }

// The same over finite floats (no NaN reaches them), as a uniform value.
template <bool MIN>
__device__ __forceinline__ float wave_reduce_f(float x) {
  const int id = __float_as_int(MIN ? __builtin_inff() : -__builtin_inff());
  auto op = [](float a, float b) { return MIN ? __builtin_fminf(a, b) : __builtin_fmaxf(a, b); };
  auto dpp = [&](float v, auto ctrl, auto rmask) {
    return __int_as_float(__builtin_amdgcn_update_dpp(id, __float_as_int(v), decltype(ctrl)::value,
                                                      decltype(rmask)::value, 0xF, false));
  };
  using c111 = std::integral_constant<int, 0x111>;
  using c112 = std::integral_constant<int, 0x112>;
  using c114 = std::integral_constant<int, 0x114>;
  using c118 = std::integral_constant<int, 0x118>;
  using c142 = std::integral_constant<int, 0x142>;
  using c143 = std::integral_constant<int, 0x143>;
  using mF = std::integral_constant<int, 0xF>;
  using mA = std::integral_constant<int, 0xA>;
  using mC = std::integral_constant<int, 0xC>;
  x = op(x, dpp(x, c111{}, mF{}));   // row_shr:1
  x = op(x, dpp(x, c112{}, mF{}));   // row_shr:2
  x = op(x, dpp(x, c114{}, mF{}));   // row_shr:4
  x = op(x, dpp(x, c118{}, mF{}));   // row_shr:8
  x = op(x, dpp(x, c142{}, mA{}));   // row_bcast:15
  x = op(x, dpp(x, c143{}, mC{}));   // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// The scores of one (row, head), all loads issued together (indices past NB
// read the last page's score and are then dropped, so no load is predicated).
// An empty window (NB = 0) reads nothing: every page is then dead.
// Blocks of 64 pages every row of NB pages fills when a kernel with PER
// blocks per lane runs it: the launch picks the smallest PER in {4, 8, 16,
// 32, 64} with 64 PER >= NB, so for PER >= 8 the first PER / 2 are full.
template <int PER>
constexpr int kFullBlocks = PER >= 8 ? PER / 2 : 0;

// The full blocks load at fixed offsets from one lane address; the others
// clamp to the last page (and are dropped as dead past NB).
template <int PER>
__device__ __forceinline__ void load_scores(const SArgs& a, int64_t r, int h, int lane, float (&v)[PER]) {
  if (a.NB <= 0) {
#pragma unroll
    for (int m = 0; m < PER; ++m) v[m] = -__builtin_inff();
    return;
  }
  const float* srow = a.bs + r * a.bs_row_stride + (int64_t)h * a.bs_head_stride;
  const float* lp = srow + lane;
#pragma unroll
  for (int m = 0; m < PER; ++m) v[m] = m < kFullBlocks<PER> ? lp[64 * m] : srow[min(64 * m + lane, a.NB - 1)];
}

// Inclusive prefix sum over the wave's lanes; declared below.
__device__ __forceinline__ uint32_t wave_scan(uint32_t x);

// Inclusive prefix sum over the wave's lanes (DPP row shifts, then the
// row-15 and row-31 broadcasts carry each row's total into the next rows).
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);   // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return x;
}

// The largest T with count(keys >= T) >= keff, over the bits below the first
// 32 - nbits (T starts from those leading bits), found 6 bits per round: the keys that share T's
// bits fixed so far are counted per next digit in the wave's LDS histogram
// (64 bins, LDS atomics), and the digit is the largest whose count, with
// every key already above, reaches keff. Lane l reads the bin of digit
// 63 - l, so an inclusive scan over the lanes counts the keys at or above
// each digit, and the first lane where that reaches keff names it. Zero keys
// (empty slots) are never counted. Against a bitwise search (one ballot round
// per bit, about 24 here) this took the top-64 selection over 4096 x 64 x
// 1024 block scores from 571 us to 509 us on one MI355X (8-bit digits:
// 521 us).
template <int N>
__device__ __forceinline__ uint32_t radix_threshold(const uint32_t (&k)[N], uint32_t T0, int nbits, uint32_t keff,
                                                    uint32_t* hist, int lane) {
  uint32_t above = 0;   // keys above every value the search can still reach
  if (nbits < 32) {
#pragma unroll
    for (int q = 0; q < N; ++q) above += ballot_count((k[q] >> nbits) > (T0 >> nbits));
  }
  uint32_t prefix = T0;
  for (int rem = nbits; rem > 0;) {
    const int w = rem < 6 ? rem : 6;
    const int sh = rem - w;
    wave_lds_sync();   // the last round's reads of the histogram are done
    hist[lane] = 0u;
    wave_lds_sync();
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const uint32_t kq = k[q];
      const bool match = kq != 0u && (rem == 32 || (kq >> rem) == (prefix >> rem));
      if (match) atomicAdd(hist + ((kq >> sh) & ((1u << w) - 1u)), 1u);
    }
    wave_lds_sync();
    const uint32_t hv = hist[63 - lane];   // lane l: digit 63 - l
    const uint32_t incl = wave_scan(hv);
    const uint64_t hit = __ballot(above + incl >= keff);
    const int L = (int)__builtin_ctzll(hit);
    above = (uint32_t)__builtin_amdgcn_readlane((int)(above + incl - hv), L);
    prefix |= (uint32_t)(63 - L) << sh;
    rem = sh;
  }
  return prefix;
}

// Emit, in page order, the keys above T and the first need_eq keys equal to
// T: page ids go to sel[] (LDS) while k fits, else straight to the output row.
template <int N>
__device__ __forceinline__ uint32_t emit(const uint32_t (&k)[N], const int32_t (&idx)[N], uint32_t T, uint32_t need_eq,
                                         int32_t* sel, int32_t* orow) {
  uint32_t written = 0, eq_seen = 0;
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const bool eq = k[q] == T;
    const uint64_t beq = __ballot(eq);
    const bool take = k[q] > T || (eq && eq_seen + lanes_below(beq) < need_eq);
    const uint64_t bt = __ballot(take);
    if (take) (sel ? sel : orow)[written + lanes_below(bt)] = idx[q];
    written += __builtin_popcountll(bt);
    eq_seen += __builtin_popcountll(beq);
  }
  return written;
}

constexpr int kSelectCand = 512;   // candidates per (row, head) the pruned search holds (8 per lane)

// Search and emit over the ncand candidates compacted in LDS (page order:
// score bits and page index), NC per lane: candidate 64 q + lane. Their keys
// are made here, the tail page's the largest.
template <int NC>
__device__ __forceinline__ uint32_t select_candidates(const uint32_t* ck, const uint16_t* ci, uint32_t ncand, int lane,
                                                      int tail, uint32_t T0, int nbits, uint32_t keff, int32_t* sel,
                                                      int32_t* orow, uint32_t* hist) {
  uint32_t k2[NC];
  int32_t i2[NC];
#pragma unroll
  for (int q = 0; q < NC; ++q) {
    const uint32_t c = 64 * q + lane;
    const int32_t j = c < ncand ? (int32_t)ci[c] : -1;
    k2[q] = c < ncand ? (j == tail ? 0xFFFFFFFFu : order_key_bits(ck[c])) : 0u;
    i2[q] = j;
  }
  const uint32_t T = radix_threshold(k2, T0, nbits, keff, hist, lane);
  uint32_t gt = 0;
#pragma unroll
  for (int q = 0; q < NC; ++q) gt += ballot_count(k2[q] > T);
  return emit(k2, i2, T, keff - gt, sel, orow);
}
constexpr int kSelectStage = 256;  // results staged in LDS for one coalesced store when k fits

// Candidates per wave the LDS holds: every score for up to 1024 pages, 512
// for longer rows (beyond, the search runs on the registers).
template <int PER>
constexpr int kCandCap = PER <= 16 ? 64 * PER : kSelectCand;

template <int PER, bool TWO>
__global__ void __launch_bounds__(kThreads) k_select(SArgs a) {
  constexpr int CAP = kCandCap<PER>;
  __shared__ uint32_t cand_keys[kWaves][CAP];     // score bits
  __shared__ uint16_t cand_idx[kWaves][CAP];      // page index (< 4096)
  __shared__ int32_t sel_all[kWaves][kSelectStage];
  __shared__ uint32_t hist_all[kWaves][64];   // radix threshold histogram
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t wave = (int64_t)blockIdx.x * kWaves + wv;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  uint32_t* ck = cand_keys[wv];
  uint16_t* ci = cand_idx[wv];
  int32_t* sel = a.k <= kSelectStage ? sel_all[wv] : nullptr;
  // Item = row * H + head. The grid stride nw is fixed, so (row, head) is
  // advanced by (nw / H, nw % H) with a carry instead of dividing per item
  // (a 64-bit division is a long scalar sequence).
  const int64_t step_r = nw / a.H;
  const int step_h = (int)(nw - step_r * a.H);
  int64_t nr = wave / a.H;
  int nh = (int)(wave - nr * a.H);
  auto advance = [&]() {
    nh += step_h;
    nr += step_r;
    if (nh >= a.H) {
      nh -= a.H;
      ++nr;
    }
  };
  // the next item's scores are in flight while this one is selected
  float nxt[PER];
  if (wave < a.items) load_scores<PER>(a, nr, nh, lane, nxt);
  for (int64_t item = wave; item < a.items; item += nw) {
    float cur[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) cur[m] = nxt[m];
    const int64_t r = nr;
    const int h = nh;
    advance();
    if (item + nw < a.items) load_scores<PER>(a, nr, nh, lane, nxt);
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

    // Per score, in floats: a dead page (-inf, or past the window: only the
    // blocks that are not surely full can reach past NB) becomes -inf, each
    // lane keeps its
    // largest score (and, for k above 64, its second largest) and counts its
    // live ones. Integer keys are made only for the candidates below.
    // The window width is opaque to the optimizer here: hoisted out of the
    // item loop, its lane mask would be spilled and reloaded for every item.
    int nb = a.NB;
    asm volatile("" : "+s"(nb));
    const float ninf = -__builtin_inff();
    float t1 = ninf, t2 = ninf;
    uint32_t live_lane = 0;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const bool fin = __builtin_isfinite(cur[m]) && (m < kFullBlocks<PER> || 64 * m + lane < nb);
      cur[m] = fin ? cur[m] : ninf;
      live_lane += fin ? 1u : 0u;
      if constexpr (TWO) t2 = __builtin_fmaxf(t2, __builtin_fminf(t1, cur[m]));
      t1 = __builtin_fmaxf(t1, cur[m]);
    }
    const uint32_t live = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(live_lane), 63);
    // the tail page is chosen whenever it is live
    const int mt = tail >> 6, lt = tail & 63;
    bool tail_live = false;
    if (tail >= 0) {
#pragma unroll
      for (int m = 0; m < PER; ++m)
        if (m == mt) tail_live = __ballot(lane == lt && cur[m] != ninf) != 0;
    }
    const uint32_t keff = min((uint32_t)a.k, live);

    int32_t* orow = a.out + r * a.out_row_stride + (int64_t)h * a.out_head_stride;
    uint32_t written = 0;
    if (keff > 0) {
      if (tail_live && keff == 1) {
        // only the tail page
        if (sel) { if (lane == 0) sel[0] = tail; } else if (lane == 0) orow[0] = tail;
        written = 1;
      } else {
        // lower bound x of the k-th largest score: the smallest lane maximum
        // when keff <= n1 lanes hold a live score (each holds one >= it),
        // else the smallest second-largest when keff <= 2 n2, else none.
        const uint32_t n1 = ballot_count(t1 != ninf);
        float x = keff <= n1 ? wave_reduce_f<true>(t1 != ninf ? t1 : __builtin_inff()) : -__FLT_MAX__;
        if constexpr (TWO) {
          if (keff > n1) {
            const uint32_t n2 = ballot_count(t2 != ninf);
            if (keff <= 2 * n2) x = wave_reduce_f<true>(t2 != ninf ? t2 : __builtin_inff());
          }
        }
        // every candidate but the tail lies in [x, K]: the search only runs
        // over the key bits below the prefix that x and K share
        const uint32_t xk = order_key(x), K = order_key(wave_reduce_f<false>(t1));
        const uint32_t diff = xk ^ K;
        const int nbits = diff ? 32 - __builtin_clz(diff) : 0;
        const uint32_t T0 = nbits == 32 ? 0u : (xk & ~((1u << nbits) - 1u));
        // candidates (scores >= x, and the tail) compacted in page order
        // (rows of up to 512 pages are searched in registers directly)
        uint32_t ncand = 0;
#pragma unroll
        for (int m = 0; m < (PER > kSelectCand / 64 ? PER : 0); ++m) {
          bool c = cur[m] >= x;
          if (m == mt) c = c || (tail_live && lane == lt);
          const uint64_t bc = __ballot(c);
          const uint32_t at = ncand + lanes_below(bc);
          if (c && (CAP >= 64 * PER || at < (uint32_t)CAP)) {
            ck[at] = __float_as_uint(cur[m]);
            ci[at] = (uint16_t)(64 * m + lane);
          }
          ncand += __builtin_popcountll(bc);
        }
        if (PER > kSelectCand / 64 && ncand <= (uint32_t)kSelectCand) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          // the candidates back in registers, as few per lane as they need
          if (ncand <= 128)
            written = select_candidates<2>(ck, ci, ncand, lane, tail, T0, nbits, keff, sel, orow, hist_all[wv]);
          else if (ncand <= 256)
            written = select_candidates<4>(ck, ci, ncand, lane, tail, T0, nbits, keff, sel, orow, hist_all[wv]);
          else
            written = select_candidates<8>(ck, ci, ncand, lane, tail, T0, nbits, keff, sel, orow, hist_all[wv]);
        } else {
          // short rows, or too many candidates: search the registers
          uint32_t key[PER];
          int32_t idx[PER];
#pragma unroll
          for (int m = 0; m < PER; ++m) {
            idx[m] = 64 * m + lane;
            key[m] = cur[m] == ninf ? 0u : order_key(cur[m]);
            if (m == mt) key[m] = (tail_live && lane == lt) ? 0xFFFFFFFFu : key[m];
          }
          const uint32_t T = radix_threshold(key, T0, nbits, keff, hist_all[wv], lane);
          uint32_t gt = 0;
#pragma unroll
          for (int m = 0; m < PER; ++m) gt += ballot_count(key[m] > T);
          written = emit(key, idx, T, keff - gt, sel, orow);
        }
      }
    }
    if (sel) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int p = lane; p < a.k; p += 64) orow[p] = (uint32_t)p < written ? sel[p] : -1;
    } else {
      for (uint32_t p = written + lane; p < (uint32_t)a.k; p += 64) orow[p] = -1;
    }
  }
}

}  // namespace

hipError_t launch_select(int per, int64_t grid, const SArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<SArgs*>(&a)};
  // the second-largest lane keys only bound the search when k exceeds the 64 lanes
  const bool two = a.k > 64;
  const void* fn = per <= 4    ? (two ? reinterpret_cast<const void*>(&k_select<4, true>)
                                      : reinterpret_cast<const void*>(&k_select<4, false>))
                   : per <= 8  ? (two ? reinterpret_cast<const void*>(&k_select<8, true>)
                                      : reinterpret_cast<const void*>(&k_select<8, false>))
                   : per <= 16 ? (two ? reinterpret_cast<const void*>(&k_select<16, true>)
                                      : reinterpret_cast<const void*>(&k_select<16, false>))
                   : per <= 32 ? (two ? reinterpret_cast<const void*>(&k_select<32, true>)
                                      : reinterpret_cast<const void*>(&k_select<32, false>))
                               : (two ? reinterpret_cast<const void*>(&k_select<64, true>)
                                      : reinterpret_cast<const void*>(&k_select<64, false>));
  return hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(kThreads), args, 0, stream);
}

}  // namespace mxs
