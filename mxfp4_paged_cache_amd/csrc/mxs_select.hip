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

// Blocks of 64 pages every row of NB pages fills when a kernel with PER
// blocks per lane runs it: the launch picks the smallest PER in {4, 8, 16,
// 32, 64} with 64 PER >= NB, so for PER >= 8 the first PER / 2 are full.
template <int PER>
constexpr int kFullBlocks = PER >= 8 ? PER / 2 : 0;

// The scores of one (row, head), all loads issued together, through buffer
// resources that end at NB: a load past NB returns 0 without reading memory
// (such pages are dropped as dead), so an empty window (NB = 0) reads nothing.
// One resource per 16 blocks keeps every offset in the instruction's 12-bit
// immediate, which the hardware's range check covers.
template <int PER>
__device__ __forceinline__ void load_scores(const float* srow, int NB, int lane, float (&v)[PER]) {
  const uint32_t bytes = NB > 0 ? 4u * (uint32_t)NB : 0u;
#pragma unroll
  for (int g = 0; g < (PER + 15) / 16; ++g) {
    const uint32_t lo = 4096u * (uint32_t)g;
    const rsrc_t rs = buffer_rsrc(srow + 1024 * g, bytes > lo ? bytes - lo : 0u);
#pragma unroll
    for (int m = 16 * g; m < min(PER, 16 * g + 16); ++m)
      v[m] = __builtin_bit_cast(float, buffer_load4_nt(rs, 4u * (uint32_t)lane + 256u * (uint32_t)(m - 16 * g)));
  }
}

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
// 32 - nbits (T starts from those leading bits), found 6 bits per round: the
// keys that share T's bits fixed so far are counted per next digit in the
// wave's LDS histogram
// (64 bins, LDS atomics), and the digit is the largest whose count, with
// every key already above, reaches keff. Lane l reads the bin of digit
// 63 - l, so an inclusive scan over the lanes counts the keys at or above
// each digit, and the first lane where that reaches keff names it. Zero keys
// (empty slots) are never counted. Against a bitwise search (one ballot round
// per bit, about 24 here) this took the top-64 selection over 4096 x 64 x
// 1024 block scores from 571 us to 509 us on one MI355X (8-bit digits:
// 521 us). When the keys at or above the chosen digit number exactly keff,
// the search stops there (on continuous scores the buckets soon hold one key
// each, so most rows skip their last rounds: 274 -> 238 us on that
// selection).
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
    const uint32_t at_or_above = (uint32_t)__builtin_amdgcn_readlane((int)(above + incl), L);
    above = (uint32_t)__builtin_amdgcn_readlane((int)(above + incl - hv), L);
    prefix |= (uint32_t)(63 - L) << sh;
    rem = sh;
    // Exactly keff keys at or above the chosen digit's bucket: the result is
    // all of them, whatever the bits below, so T is just below the bucket.
    if (at_or_above == keff && rem > 0 && prefix != 0u) return prefix - 1u;
  }
  return prefix;
}

// Emit, in page order, the keys above T and the first need_eq keys equal to
// T: page ids go to sel[] (LDS) while k fits, else straight to the output row.
template <int N>
__device__ __forceinline__ uint32_t emit(const uint32_t (&k)[N], const int32_t (&idx)[N], uint32_t T, uint32_t need_eq,
                                         int32_t* sel, int32_t* orow) {
  uint32_t written = 0, eq_seen = 0;
  if (need_eq == 0u) {   // nothing taken at T (the search stopped on a bucket edge)
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const bool take = k[q] > T;
      const uint64_t bt = __ballot(take);
      if (take) (sel ? sel : orow)[written + lanes_below(bt)] = idx[q];
      written += __builtin_popcountll(bt);
    }
    return written;
  }
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

constexpr int kSelectCand = 512;   // candidates per (row, head) the LDS holds (8 per lane)
constexpr int kSelectStage = 256;  // results staged in LDS for one coalesced store when k fits

// Per-wave LDS block of the candidates: score bits at [0, CAP), page indices
// at [kIdxOff, kIdxOff + CAP), so one ds_write2st64 / ds_read2st64 moves both
// (kIdxOff is a multiple of 64 dwords). Slots [CAP, CAP + 64) of each half
// take the writes of lanes that hold no candidate (one per lane, so no two
// lanes of a store meet). The staged results reuse the block's first dwords:
// they are written only after every candidate is back in registers.
constexpr int kCandPad = kSelectCand + 64;
constexpr int kIdxOff = kCandPad;
static_assert(kIdxOff % 64 == 0, "the index half must sit a whole number of 64-dword rows on");
static_assert(kSelectStage <= kSelectCand, "the result stage must fit in the candidate block");

// Search and emit over the ncand candidates compacted in LDS in page order,
// NC per lane: candidate 64 q + lane. Their keys are made here, the tail
// page's the largest. Slots past ncand hold stale values and are dropped.
template <int NC>
__device__ __forceinline__ uint32_t select_candidates(const uint32_t* cb, uint32_t ncand, int lane, int tail,
                                                      uint32_t T0, int nbits, uint32_t keff, int32_t* sel,
                                                      int32_t* orow, uint32_t* hist) {
  uint32_t k2[NC];
  int32_t i2[NC];
#pragma unroll
  for (int q = 0; q < NC; ++q) {
    const uint32_t c = 64 * q + lane;
    uint32_t bits = cb[c];
    int32_t j = (int32_t)cb[kIdxOff + c];
    // every slot is read (stale ones are dropped here); without this the
    // compiler turns each read into a branch around it
    asm volatile("" : "+v"(bits), "+v"(j));
    k2[q] = c < ncand ? (j == tail ? 0xFFFFFFFFu : order_key_bits(bits)) : 0u;
    i2[q] = c < ncand ? j : -1;
  }
  const uint32_t T = radix_threshold(k2, T0, nbits, keff, hist, lane);
  uint32_t gt = 0;
#pragma unroll
  for (int q = 0; q < NC; ++q) gt += ballot_count(k2[q] > T);
  return emit(k2, i2, T, keff - gt, sel, orow);
}

// Scores per lane at which rows stop being searched on the registers directly
// and candidates are compacted first (rows of up to 512 pages are searched in
// registers).
constexpr int kCompactPer = kSelectCand / 64;

// Waves per SIMD the register budget is set for: eight hide the load
// latency of rows up to 1024 pages; longer rows hold more scores per lane.
template <int PER>
constexpr int kSelectWaves = PER <= 16 ? 8 : (PER == 32 ? 4 : 2);

template <int PER, bool TWO>
__global__ void __launch_bounds__(kThreads, kSelectWaves<PER>) k_select(SArgs a) {
  constexpr int CAP = kSelectCand;
  __shared__ uint32_t cand_all[kWaves][2 * kCandPad];
  __shared__ uint32_t hist_all[kWaves][64];   // radix threshold histogram
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t wave = (int64_t)blockIdx.x * kWaves + wv;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  uint32_t* cb = cand_all[wv];
  int32_t* sel = a.k <= kSelectStage ? reinterpret_cast<int32_t*>(cb) : nullptr;
  // Item = row * H + head. The grid stride nw is fixed, so (row, head) is
  // advanced by (nw / H, nw % H) with a carry instead of dividing per item
  // (a 64-bit division is a long scalar sequence).
  const int64_t step_r = nw / a.H;
  const int step_h = (int)(nw - step_r * a.H);
  int64_t r = wave / a.H;
  int h = (int)(wave - r * a.H);
  // The waves per SIMD hide the load latency; prefetching the next item's
  // scores would cost PER more registers per lane and measured slower.
  for (int64_t item = wave; item < a.items; item += nw) {
    // The lane index is opaque to the optimizer inside the loop: hoisted,
    // each page index and offset derived from it (64 m + lane, ...) would
    // hold a register of its own for the whole loop and push the kernel
    // past the register budget.
    int lane = (int)threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    float cur[PER];
    const float* srow = a.bs + r * a.bs_row_stride + (int64_t)h * a.bs_head_stride;
    load_scores<PER>(srow, a.NB, lane, cur);
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
      lim = causal_limit(a.seq[lo], a.prefix[lo], (int)(r - a.cu[lo]));
    }
    lim = clampi(lim, 0, a.max_seq_len);
    const int tail = lim > 0 ? (lim - 1) / a.P : -1;
    int32_t* orow = a.out + r * a.out_row_stride + (int64_t)h * a.out_head_stride;
    h += step_h;
    r += step_r;
    if (h >= a.H) {
      h -= a.H;
      ++r;
    }

    // Per score, in floats: a dead page (-inf, or past the window: only the
    // blocks that are not surely full can reach past NB) becomes -inf and
    // each lane keeps its largest score (and, for k above 64, its second
    // largest). Integer keys are made only for the candidates below.
    // The window width is opaque to the optimizer here: hoisted out of the
    // item loop, its lane mask would be spilled and reloaded for every item.
    int nb = a.NB;
    asm volatile("" : "+s"(nb));
    const float ninf = -__builtin_inff();
    float t1 = ninf, t2 = ninf;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const bool fin = __builtin_isfinite(cur[m]) && (m < kFullBlocks<PER> || lane < nb - 64 * m);
      cur[m] = fin ? cur[m] : ninf;
      if constexpr (TWO) t2 = __builtin_fmaxf(t2, __builtin_fminf(t1, cur[m]));
      t1 = __builtin_fmaxf(t1, cur[m]);
    }
    // live pages: at least n1 (the lanes holding one), counted exactly only
    // when that many might fall short of k
    const uint32_t n1 = ballot_count(t1 != ninf);
    uint32_t live = n1;
    if (n1 < (uint32_t)a.k) {
      live = 0;
#pragma unroll
      for (int m = 0; m < PER; ++m) live += ballot_count(cur[m] != ninf);
    }
    const uint32_t keff = min((uint32_t)a.k, live);

    uint32_t written = 0;
    if (keff > 0) {
      // lower bound x of the k-th largest key: the smallest lane maximum
      // when keff <= n1 lanes hold a live score (each holds one >= it),
      // else the smallest second-largest when keff <= 2 n2, else none
      // (the key of the lowest finite score). Reduced as keys.
      constexpr uint32_t kLowestKey = 0x00800001u;   // key of -FLT_MAX
      const uint32_t k1 = t1 != ninf ? order_key(t1) : 0u;
      uint32_t xk = keff <= n1 ? wave_min(k1 != 0u ? k1 : 0xFFFFFFFFu) : kLowestKey;
      if constexpr (TWO) {
        if (keff > n1) {
          const uint32_t k2 = t2 != ninf ? order_key(t2) : 0u;
          if (keff <= 2 * ballot_count(k2 != 0u)) xk = wave_min(k2 != 0u ? k2 : 0xFFFFFFFFu);
        }
      }
      // every candidate but the tail lies in [x, K] (K the largest lane
      // maximum; the tail's key is raised to the largest): the search only
      // runs over the key bits below the prefix that x and K share
      const uint32_t K = wave_max(k1);
      const uint32_t diff = xk ^ K;
      const int nbits = diff ? 32 - __builtin_clz(diff) : 0;
      const uint32_t T0 = nbits == 32 ? 0u : (xk & ~((1u << nbits) - 1u));
      const int mt = tail >> 6, lt = tail & 63;
      bool done = false;
      if (PER > kCompactPer) {
        // Candidates compacted in page order: the scores >= x and, on the
        // tail's lane, every live score, so the tail is among them whatever
        // its score (its key is raised when they are read back; the others
        // of that lane fall below T if they are below x).
        const float x = __uint_as_float((xk & 0x80000000u) ? (xk & 0x7FFFFFFFu) : 0u - xk);
        const float xl = (tail >= 0 && lane == lt) ? -__FLT_MAX__ : x;
        // the last item's staged results (which share this block) are read
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        uint32_t ncand = 0;
        const uint32_t spare = (uint32_t)(CAP + lane);
#pragma unroll
        for (int m = 0; m < (PER > kCompactPer ? PER : 0); ++m) {
          const bool c = cur[m] >= xl;
          const uint64_t bc = __ballot(c);
          const uint32_t at = __builtin_amdgcn_mbcnt_hi((uint32_t)(bc >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)bc, ncand));
          uint32_t* cw = cb + min(c ? at : 0xFFFFFFFFu, spare);
          cw[0] = __float_as_uint(cur[m]);
          cw[kIdxOff] = (uint32_t)(64 * m + lane);
          ncand += __builtin_popcountll(bc);
        }
        if (ncand <= (uint32_t)CAP) {
          done = true;
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          // the candidates back in registers, as few per lane as they need
          // (every step of 64 has its own variant: the search and the emit
          // cost per register held, and rounding 257 candidates up to eight
          // per lane cost 5% of the top-64 selection)
          if (ncand <= 64)
            written = select_candidates<1>(cb, ncand, lane, tail, T0, nbits, keff, sel, orow, hist_all[wv]);
          else if (ncand <= 128)
            written = select_candidates<2>(cb, ncand, lane, tail, T0, nbits, keff, sel, orow, hist_all[wv]);
          else if (ncand <= 192)
            written = select_candidates<3>(cb, ncand, lane, tail, T0, nbits, keff, sel, orow, hist_all[wv]);
          else if (ncand <= 256)
            written = select_candidates<4>(cb, ncand, lane, tail, T0, nbits, keff, sel, orow, hist_all[wv]);
          else if (ncand <= 320)
            written = select_candidates<5>(cb, ncand, lane, tail, T0, nbits, keff, sel, orow, hist_all[wv]);
          else if (ncand <= 384)
            written = select_candidates<6>(cb, ncand, lane, tail, T0, nbits, keff, sel, orow, hist_all[wv]);
          else if (ncand <= 448)
            written = select_candidates<7>(cb, ncand, lane, tail, T0, nbits, keff, sel, orow, hist_all[wv]);
          else
            written = select_candidates<8>(cb, ncand, lane, tail, T0, nbits, keff, sel, orow, hist_all[wv]);
        }
      }
      if (!done) {
        // short rows, or too many candidates: search the registers (dead
        // pages key 0, a live tail the largest key)
        uint32_t key[PER];
        int32_t idx[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
          idx[m] = 64 * m + lane;
          key[m] = cur[m] == ninf ? 0u : order_key(cur[m]);
          if (m == mt) key[m] = (lane == lt && key[m] != 0u) ? 0xFFFFFFFFu : key[m];
        }
        const uint32_t T = radix_threshold(key, T0, nbits, keff, hist_all[wv], lane);
        uint32_t gt = 0;
#pragma unroll
        for (int m = 0; m < PER; ++m) gt += ballot_count(key[m] > T);
        written = emit(key, idx, T, keff - gt, sel, orow);
      }
    }
    if (sel) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // non-temporal: the ids are not read back here (231 -> 225 us for top-64
      // over 4096 x 64 x 1024 block scores)
      for (int p = lane; p < a.k; p += 64) __builtin_nontemporal_store((uint32_t)p < written ? sel[p] : -1, orow + p);
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
