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
// fp8 cache) and read by all four waves. Block scores are staged in LDS for up to 16 pages and leave as
// contiguous per-slot rows.
//
// Work items are ordered slot block fastest: at any moment the whole grid
// works on one chunk of pages (small enough for every XCD's L2), and each
// workgroup's items are spread over all query rows and all chunks, so the
// causal triangle (chunks past some rows' limits are cheap) costs every
// workgroup the same.
// ---------------------------------------------------------------------------
constexpr int kPrefillSlots = kWaves * kPrefillTiles * 16;   // query slots per work item
constexpr int kPrefillStagePages = 16;                        // pages per block-score flush
constexpr int kPrefillStageStride = kPrefillStagePages + 1;   // LDS row pitch (odd: no bank conflicts)
constexpr int kFlushLanesPerRow = kPrefillStagePages / 4;     // 4 pages per lane

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
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i = lane & 15;
  const float s = a.sm_scale;

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
    const int item_lim = clampi(min(seq, pre + (int)(slast / a.H) + 1), 0, a.max_seq_len);

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
      lim[n] = valid ? clampi(min(seq, pre + r + 1), 0, a.max_seq_len) : 0;
      qt[n] = load_q_tile_masked<QDT>(a.q + grow * a.q_row_stride + (int64_t)h * a.q_head_stride, g, valid);
    }
    // smallest limit among this wave's slots: the limit of its first slot
    const int64_t wfirst = sbeg + (int64_t)wave * NQ * 16;
    const int wave_min_lim = wfirst < nslots ? clampi(min(seq, pre + (int)(wfirst / a.H) + 1), 0, a.max_seq_len) : 0;

    const int j0 = pc * a.pages_per_item;
    const int j1 = min(j0 + a.pages_per_item, a.NB);
    const int jl = min(j1, (item_lim + P - 1) / P);   // pages [j0, jl) hold live tokens
    const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;

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
    int jbase = j0;
    for (int j = j0; j < j1; ++j) {
      float r[NQ];
      if (j < jl) {
        const bool more = j + 1 < jl;
        PageStage<KDT, P> nx;
        if (more) {
          if (j + 1 - jid == 64) {
            jid += 64;
            ids = (jid + lane < jl) ? btrow[jid + lane] : 0;
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
      {
        if (g == 0) {
#pragma unroll
          for (int n = 0; n < NQ; ++n) stage[((wave * NQ + n) * 16 + i) * kPrefillStageStride + (j - jbase)] = r[n] * s;
        }
        if ((j + 1) % kPrefillStagePages == 0 || j == j1 - 1) {
          // Each wave flushes its own slot rows [wave * 16 NQ, +16 NQ) for pages
          // [jbase, j]; no other wave touches them, so no workgroup barrier is
          // needed (a wave's LDS accesses complete in order; the fences keep the
          // compiler from moving its reads above its writes). A group of TPR
          // lanes writes one contiguous run of a row, 4 pages per lane; windows
          // end at multiples of the window size, so in aligned rows a full
          // window covers whole 64- or 128-byte lines.
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const int npg = j - jbase + 1;
          constexpr int TPR = kFlushLanesPerRow;
          const int part = lane % TPR;
          const int lo = wave * NQ * 16;
          const int hi = (int)min((int64_t)lo + NQ * 16, nslots - sbeg);
          const bool full = 4 * part + 3 < npg;
          const bool v4 = a.vec_bs == 4 && (jbase & 3) == 0 && full;
          const bool v2 = a.vec_bs >= 2 && (jbase & 1) == 0 && full;
          const uint32_t slot0 = (uint32_t)(sbeg - (int64_t)(a.H) * (sbeg / a.H));   // slot sbeg within its row
          const int64_t rowb = (int64_t)row0 + sbeg / a.H;
          for (int sl = lo + lane / TPR; sl < hi; sl += 64 / TPR) {
            if (4 * part >= npg) continue;
            const uint32_t slot = slot0 + (uint32_t)sl;
            const uint32_t dr = slot / (uint32_t)a.H;
            float* dst = a.bs + (rowb + dr) * a.bs_row_stride + (int64_t)(slot - dr * (uint32_t)a.H) * a.bs_head_stride +
                         jbase + 4 * part;
            const float* src = stage + sl * kPrefillStageStride + 4 * part;
            if (v4) {
              const v4f v = {src[0], src[1], src[2], src[3]};
              *reinterpret_cast<v4f*>(dst) = v;
            } else if (v2) {
              typedef float v2f __attribute__((ext_vector_type(2)));
              const v2f v0 = {src[0], src[1]}, v1 = {src[2], src[3]};
              reinterpret_cast<v2f*>(dst)[0] = v0;
              reinterpret_cast<v2f*>(dst)[1] = v1;
            } else {
              for (int x = 0; x < 4 && 4 * part + x < npg; ++x) dst[x] = src[x];
            }
          }
          jbase = j + 1;
        }
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
