// Prefill block-score kernel of the paged MXFP4 index scorer (gfx950).
// Compiled without NaN semantics for float arithmetic (see the build): the
// kernel only compares and folds finite scores and -inf.
#include "mxs_device.h"

namespace mxs {
namespace {
using namespace dev;

// ---------------------------------------------------------------------------
// Prefill block scores: one workgroup per work item (request, block of 512
// query slots, chunk of pages), looping over items with a grid stride. A
// query slot is (row, head); slot = row * H + head, so a 16-slot tile is 16
// heads of one row when H is a multiple of 16. Each wave keeps 8 query tiles
// in registers for the whole item; every page is staged once per workgroup in
// LDS (double-buffered, 8.5 KB per buffer at P = 128 for MXFP4, 16 KB for an
// fp8 cache) and read by all four waves. Block scores are staged in an LDS
// ring of 16 pages per slot and leave as 64-byte-aligned segments of each
// output row (see the flush below).
//
// Work items are ordered slot block fastest: at any moment the whole grid
// works on one chunk of pages (small enough for every XCD's L2), and each
// workgroup's items are spread over all query rows and all chunks, so the
// causal triangle (chunks past some rows' limits are cheap) costs every
// workgroup the same.
// ---------------------------------------------------------------------------
// A float in global memory: the flush's row pointers come back from LDS as
// plain integers, and as generic pointers their stores were flat stores,
// whose completion the LDS waits of the next page also waited for.
typedef __attribute__((address_space(1))) float gfloat;
constexpr int kPrefillSlots = kWaves * kPrefillTiles * 16;   // query slots per work item
constexpr int kWaveSlots = kPrefillTiles * 16;                // query slots per wave
constexpr int kRingPages = 16;                                // block scores per slot in the LDS ring: 64 bytes
constexpr int kPrefillStageStride = kRingPages + 1;           // LDS row pitch (odd: no bank conflicts)

// Score one LDS-resident page against this wave's query tiles; r[n] gets the
// (unscaled) max over the page's live tokens for slot (tile n, lane i).
//
// Software-pipelined over the page's 16-token tiles: a step
// reads the next tile's K operand from LDS, then issues the NQ MFMAs of tile
// t, each followed by the fold (two v_max3) of the matching result of tile
// t - 1. A fold thus reads a result written NQ MFMAs earlier, past the
// MFMA-to-VALU hazard window, so no wait states sit between them (with each
// fold right behind its own MFMA, every other MFMA was padded with 9 wait
// states). Two result sets alternate between the halves of a loop trip, so
// only two tiles of results are live and none is copied.
template <int KDT, int P, int NQ, bool MASK>
__device__ __forceinline__ void prefill_page(const uint8_t* kb, const v8i (&qt)[NQ], const int (&lrel)[NQ], int g,
                                             int i, float (&r)[NQ]) {
  constexpr int TPP = P / 16;
  // The masked and unmasked variants begin alike (the first tile is not
  // folded yet); this marker keeps the compiler from hoisting that common
  // start above the branch between them, which left the first tile's results
  // in registers the unmasked loop then had to copy out of (32 moves a page).
  asm volatile("; prefill page, mask %0" ::"n"(MASK ? 1 : 0));
  float m[NQ];
#pragma unroll
  for (int n = 0; n < NQ; ++n) m[n] = kNegInf;
  auto fold1 = [&](int t, int n, v4f c) {
    if constexpr (MASK) {
#pragma unroll
      for (int v = 0; v < 4; ++v) c[v] = (16 * t + v < lrel[n]) ? c[v] : kNegInf;
    }
    m[n] = max_into(m[n], c);
  };
  // tile t's MFMAs into cur, interleaved with the folds of tile t - 1 (prev)
  // when there is one; the next tile's K reads go first
  auto step = [&](int t, const KTile<KDT>& k, v4f (&cur)[NQ], const v4f (&prev)[NQ]) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      cur[n] = mma_tile(k, qt[n]);
      if (t > 0) fold1(t - 1, n, prev[n]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                     // LDS reads of the next tile
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // one MFMA
      if (t > 0) __builtin_amdgcn_sched_group_barrier(0x002, MASK ? 6 : 2, 0);   // one fold
    }
  };
  v4f cA[NQ], cB[NQ];
  // The wave issues its MFMAs at raised priority, so that of the two waves
  // sharing a SIMD the one with matrix work goes first (measured 1-2% on
  // both block-score workloads).
  __builtin_amdgcn_s_setprio(1);
  KTile<KDT> kA = lds_tile<KDT, P>(kb, g, i, 0);
  KTile<KDT> kB = lds_tile<KDT, P>(kb, g, i, 1);
  step(0, kA, cA, cB);
#pragma unroll 1
  for (int t = 1; t < TPP - 1; t += 2) {
    kA = lds_tile<KDT, P>(kb, g, i, t + 1);
    step(t, kB, cB, cA);
    kB = lds_tile<KDT, P>(kb, g, i, t + 2);
    step(t + 1, kA, cA, cB);
  }
  step(TPP - 1, kB, cB, cA);
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int n = 0; n < NQ; ++n) fold1(TPP - 1, n, cB[n]);
#pragma unroll
  for (int n = 0; n < NQ; ++n) r[n] = fold_groups(m[n]);
}

template <int QDT, int KDT, int P>
__global__ void __launch_bounds__(kThreads, 2) k_prefill(KArgs a) {
  constexpr int NQ = kPrefillTiles;
  constexpr int PB = kStagedPageBytes<KDT, P>;   // bytes of one staged page
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2 * PB];
  __shared__ float stage[kPrefillSlots * kPrefillStageStride];
  // Block-score flush bookkeeping, per wave: the output row of each of its
  // slots (address of page 0) and, per page phase e, the slots whose 64-byte
  // output segments end at pages j with j % 16 == e.
  __shared__ uint64_t frow_all[kWaves][kWaveSlots];
  __shared__ uint8_t flist_all[kWaves][kRingPages][kWaveSlots];
  __shared__ uint32_t fcount_all[kWaves][kRingPages];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i = lane & 15;
  const float s = a.sm_scale;
  uint64_t* frow = frow_all[wave];
  uint32_t* fcount = fcount_all[wave];
  float* ring = stage + wave * kWaveSlots * kPrefillStageStride;

  for (int64_t item = blockIdx.x; item < a.items; item += gridDim.x) {
    const int sb = (int)(item % a.slot_items);
    const int64_t rest = item / a.slot_items;
    const int pc = (int)(rest % a.page_items);
    const int b = (int)(rest / a.page_items);
    const int row0 = a.cu[b];
    const int qlen = a.cu[b + 1] - row0;
    const int64_t nslots = (int64_t)qlen * a.H;
    const int64_t sbeg = (int64_t)sb * kPrefillSlots;
    if (sbeg >= nslots) continue;   // uniform over the workgroup
    const int seq = a.seq[b], pre = a.prefix[b];
    const int64_t slast = min(sbeg + (int64_t)kPrefillSlots, nslots) - 1;
    const int item_lim = clampi(causal_limit(seq, pre, (int)(slast / a.H)), 0, a.max_seq_len);

    // this lane's query slots
    v8i qt[NQ];
    int lim[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const int64_t sl = sbeg + (int64_t)(wave * NQ + n) * 16 + i;
      const bool valid = sl < nslots;
      const int64_t slc = valid ? sl : nslots - 1;
      const int r = (int)(slc / a.H);
      const int h = (int)(slc % a.H);
      const int64_t grow = (int64_t)row0 + r;
      lim[n] = valid ? clampi(causal_limit(seq, pre, r), 0, a.max_seq_len) : 0;
      qt[n] = load_q_tile_masked<QDT>(a.q + grow * a.q_row_stride + (int64_t)h * a.q_head_stride, g, valid);
    }
    // smallest limit among this wave's slots: the limit of its first slot
    const int64_t wfirst = sbeg + (int64_t)wave * NQ * 16;
    const int wave_min_lim =
        wfirst < nslots ? clampi(causal_limit(seq, pre, (int)(wfirst / a.H)), 0, a.max_seq_len) : 0;

    const int j0 = pc * a.pages_per_item;
    const int j1 = min(j0 + a.pages_per_item, a.NB);
    const int jl = min(j1, (item_lim + P - 1) / P);   // pages [j0, jl) hold live tokens
    const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;

    // Output rows of this wave's slots and the phase at which each row's
    // 64-byte segments end: row element j (page j) sits at float index
    // ax + j, so a segment ends at every page j with (ax + j + 1) % 16 == 0.
    // The slots are bucketed by that phase, so each page's flush touches
    // only the rows that complete a segment there.
    const int wslots = (int)min((int64_t)kWaveSlots, max((int64_t)0, nslots - sbeg - (int64_t)wave * kWaveSlots));
    {
      const uint32_t slot0 = (uint32_t)(sbeg - (int64_t)(a.H) * (sbeg / a.H));   // slot sbeg within its row
      const int64_t rowb = (int64_t)row0 + sbeg / a.H;
      wave_lds_sync();   // the last item's flush reads are done
      if (lane < kRingPages) fcount[lane] = 0u;
      wave_lds_sync();
#pragma unroll
      for (int half = 0; half < kWaveSlots / 64; ++half) {
        const int sl = half * 64 + lane;
        if (sl < wslots) {
          const uint32_t slot = slot0 + (uint32_t)(wave * kWaveSlots + sl);
          const uint32_t dr = slot / (uint32_t)a.H;
          float* rp = a.bs + (rowb + dr) * a.bs_row_stride + (int64_t)(slot - dr * (uint32_t)a.H) * a.bs_head_stride;
          frow[sl] = reinterpret_cast<uint64_t>(rp);
          const uint32_t e = (0u - (uint32_t)(reinterpret_cast<uint64_t>(rp) >> 2) - 1u) & (kRingPages - 1);
          const uint32_t pos = atomicAdd(&fcount[e], 1u);
          flist_all[wave][e][pos] = (uint8_t)sl;
        }
      }
      wave_lds_sync();
    }
    // Write the staged scores of slot sl for the pages of its current 64-byte
    // segment (the one holding page j) from the item's first page on: lane
    // quarter q writes pages w + 4q .. w + 4q + 3, one 16-byte store when all
    // four are this item's. The stores are non-temporal: held in L2 as usual,
    // the 128-byte lines whose halves are written 16 pages apart went out to
    // memory as about 10% more bytes than the scores (counted on the 4096-row
    // prefill) and pushed the K pages the other workgroups were reading out
    // of L2 (the chunked prefill fetched 1.7x more).
    auto flush_slot = [&](int sl, int j) {
      gfloat* rp = reinterpret_cast<gfloat*>(frow[sl]);
      const uint32_t ax = (uint32_t)(reinterpret_cast<uint64_t>(rp) >> 2);
      const int p0 = j - (int)((ax + (uint32_t)j) & (kRingPages - 1)) + 4 * (lane & 3);
      const float* src = ring + sl * kPrefillStageStride;
      if (p0 >= j0 && p0 + 3 <= j) {
        const v4f v = {src[p0 & 15], src[(p0 + 1) & 15], src[(p0 + 2) & 15], src[(p0 + 3) & 15]};
        __builtin_nontemporal_store(v, reinterpret_cast<__attribute__((address_space(1))) v4f*>(rp + p0));
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (p0 + x >= j0 && p0 + x <= j) __builtin_nontemporal_store(src[(p0 + x) & 15], rp + p0 + x);
      }
    };

    // page ids, 64 at a time: lane l holds the id of page jid + l (one table
    // read per 64 pages, picked per page with readlane, so no page waits on
    // a table read before its loads can issue)
    int jid = j0;
    int ids = (j0 + lane < jl) ? btrow[j0 + lane] : 0;
    auto load_page = [&](PageStage<KDT, P>& st, int64_t page) {
      stage_load<KDT, P>(st, a.kd + page * a.kd_page_stride,
                         KDT == MXS_K_MXFP4 ? a.ks + page * a.ks_page_stride : nullptr, tid);
    };
    if (j0 < jl) {
      PageStage<KDT, P> st;
      load_page(st, __builtin_amdgcn_readfirstlane(ids));
      stage_store<KDT, P>(st, kbuf, tid);
    }
    __syncthreads();
    for (int j = j0; j < j1; ++j) {
      float r[NQ];
      if (j < jl) {
        const bool more = j + 1 < jl;
        PageStage<KDT, P> nx;
        if (more) {
          if (j + 1 - jid == 64) {
            jid += 64;
            ids = (jid + lane < jl) ? btrow[jid + lane] : 0;
            // wait for the ids here: left to the page's readlane, the wait
            // (whose counter also covers the block-score stores) went on
            // every page, since the compiler cannot tell on which ones
            // this load is in flight
            asm volatile("" ::"v"(ids));
          }
          load_page(nx, __builtin_amdgcn_readlane(ids, j + 1 - jid));
        }
        const uint8_t* kb = kbuf + ((j - j0) & 1) * PB;
        int lrel[NQ];
#pragma unroll
        for (int n = 0; n < NQ; ++n) lrel[n] = lim[n] - j * P - 4 * g;
        if ((j + 1) * P > wave_min_lim)
          prefill_page<KDT, P, NQ, true>(kb, qt, lrel, g, i, r);
        else
          prefill_page<KDT, P, NQ, false>(kb, qt, lrel, g, i, r);
        if (more) stage_store<KDT, P>(nx, kbuf + ((j + 1 - j0) & 1) * PB, tid);
      } else {
#pragma unroll
        for (int n = 0; n < NQ; ++n) r[n] = kNegInf;
      }
      if (g == 0) {
#pragma unroll
        for (int n = 0; n < NQ; ++n) ring[(n * 16 + i) * kPrefillStageStride + (j & (kRingPages - 1))] = r[n] * s;
      }
      // Each wave flushes its own slots' rows (no other wave touches them, so
      // no workgroup barrier: a wave's LDS accesses complete in order, and
      // the fences keep the compiler from moving its reads above its writes).
      // A row's segment leaves when complete, as whole 64-byte-aligned
      // pieces: with rows that are not 64-byte aligned (1038 floats each, say)
      // fixed 16-page windows split every piece over two segments, and the
      // chunked prefill took 4% longer than with aligned rows. On the item's
      // last page every slot writes what is left of its segment.
      wave_lds_sync();
      if (j == j1 - 1) {
        for (int sl = lane >> 2; sl < wslots; sl += 16) flush_slot(sl, j);
      } else {
        const uint32_t e = (uint32_t)j & (kRingPages - 1);
        const int cnt = __builtin_amdgcn_readfirstlane((int)fcount[e]);
        for (int k = lane >> 2; k < cnt; k += 16) flush_slot(flist_all[wave][e][k], j);
      }
      __syncthreads();
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

template <int QDT, int KDT, int P>
struct Launch {
  static hipError_t run(const mxs_plan& plan, const KArgs& a, hipStream_t stream) {
    void* args[] = {const_cast<KArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_prefill<QDT, KDT, P>), dim3(plan.grid), dim3(kThreads),
                           args, 0, stream);
  }
};

template <int QDT, int KDT, int P>
struct Occupancy {
  static int run() { return occ_of(&k_prefill<QDT, KDT, P>); }
};

}  // namespace

hipError_t launch_prefill(const mxs_plan& plan, const KArgs& a, hipStream_t stream) {
  return dispatch_variant<Launch>(plan.q_dtype, plan.k_dtype, plan.page_size, plan, a, stream);
}

int occupancy_prefill(int32_t q_dtype, int32_t k_dtype, int32_t page_size) {
  return dispatch_variant<Occupancy>(q_dtype, k_dtype, page_size);
}

}  // namespace mxs
