// Logits kernel of the paged MXFP4 index scorer (gfx950): per-token logits
// [rows, H, max_seq_len], optionally with the per-page block scores.
// Compiled without NaN semantics for float arithmetic (see the build): the
// kernel only compares and folds finite scores and -inf.
#include "mxs_device.h"

namespace mxs {
namespace {
using namespace dev;

// ---------------------------------------------------------------------------
// One workgroup per work item (request, block of 64 query slots, chunk of
// pages), looping over items with a grid stride; each wave holds one 16-slot
// query tile. A page is staged once per workgroup in LDS (as in prefill, for
// either cache format) and multiplied by all four waves.
//
// The output dominates this path (4 bytes per (row, head, token)), so it is
// written the way HBM takes it fastest: the MFMA results of each wave go
// through an LDS window of [16 slots][128 tokens] and leave as whole 512-byte
// row segments, two rows per store instruction. Stored straight from the MFMA
// layout, each instruction would write 64-byte pieces of 16 different rows,
// which measured at about half the write bandwidth on this chip.
//
// Work items are ordered page chunk fastest. Workgroups go round-robin over
// the 8 XCDs, so with a grid and a chunk count that are both multiples of 8,
// workgroup c only sees chunks c mod 8 and each XCD keeps one eighth of the
// pages in its own L2. When the queries outweigh the pages (xcd_split), XCD
// x instead takes the contiguous items [x items / 8, (x + 1) items / 8),
// strided over its own workgroups: its eighth of the query slots and the
// pages they are scored against.
// ---------------------------------------------------------------------------
constexpr int kLogitsSlots = kWaves * 16;   // query slots per work item
constexpr int kWinTokens = 128;             // tokens per output window: 512 bytes of a logits row
constexpr int kWinPitch = kWinTokens + 4;   // LDS row pitch in floats (16-byte pad: no bank conflicts)

template <int QDT, int KDT, int P, bool WANT_BS>
__global__ void __launch_bounds__(kThreads, 2) k_logits(KArgs a) {
  constexpr int PB = kStagedPageBytes<KDT, P>;   // bytes of one staged page
  constexpr int TPP = P / 16;              // 16-token tiles per page
  constexpr int PPW = kWinTokens / P;      // pages per output window
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2 * PB];
  __shared__ __attribute__((aligned(16))) float win_all[kWaves][16 * kWinPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i = lane & 15;
  float* win = win_all[wave];
  const float s = a.sm_scale;
  const int W = a.max_seq_len;
  const v4f ninf = {kNegInf, kNegInf, kNegInf, kNegInf};
  // write-out map: lanes 0..31 write row 2q, lanes 32..63 row 2q + 1, 16 bytes each
  const int wrow = lane >> 5, wcol = lane & 31;

  int64_t item_lo = 0, item_hi = a.items, item0 = blockIdx.x, item_step = gridDim.x;
  if (a.xcd_split) {   // the plan makes the grid a multiple of 8
    const int x = blockIdx.x & 7;
    item_lo = a.items * x / 8;
    item_hi = a.items * (x + 1) / 8;
    item0 = item_lo + (blockIdx.x >> 3);
    item_step = gridDim.x >> 3;
  }
  for (int64_t item = item0; item < item_hi; item += item_step) {
    const int pc = (int)(item % a.page_items);
    const int64_t rest = item / a.page_items;
    const int sb = (int)(rest % a.slot_items);
    const int b = (int)(rest / a.slot_items);
    // decode rows: request b is row b with one query, seeing its seq_len tokens
    const int row0 = a.decode_rows ? b : a.cu[b];
    const int qlen = a.decode_rows ? 1 : a.cu[b + 1] - row0;
    const int64_t nslots = (int64_t)qlen * a.H;
    const int64_t sbeg = (int64_t)sb * kLogitsSlots;
    if (sbeg >= nslots) continue;   // uniform over the workgroup
    const int seq = a.seq[b], pre = a.decode_rows ? seq - 1 : a.prefix[b];
    const int64_t slast = min(sbeg + (int64_t)kLogitsSlots, nslots) - 1;
    const int item_lim = clampi(causal_limit(seq, pre, (int)(slast / a.H)), 0, W);

    // the wave's tile: slots wbeg .. wbeg + 15; slot wbeg is (row r0, head h0)
    const int64_t wbeg = sbeg + (int64_t)wave * 16;
    const bool wave_live = wbeg < nslots;
    const int64_t w0 = wave_live ? wbeg : nslots - 1;
    const int r0 = (int)(w0 / a.H), h0 = (int)(w0 - (int64_t)r0 * a.H);
    // MFMA slot of this lane: wbeg + i
    const bool valid = wbeg + i < nslots;
    const uint32_t hi_ = (uint32_t)h0 + (uint32_t)(valid ? i : 0);
    const int r = r0 + (int)(hi_ / (uint32_t)a.H), h = (int)(hi_ % (uint32_t)a.H);
    const int lim = valid ? clampi(causal_limit(seq, pre, r), 0, W) : 0;
    const v8i qt =
        load_q_tile_masked<QDT>(a.q + ((int64_t)row0 + r) * a.q_row_stride + (int64_t)h * a.q_head_stride, g, valid);
    float* bsp = (WANT_BS && valid) ? a.bs + ((int64_t)row0 + r) * a.bs_row_stride + (int64_t)h * a.bs_head_stride
                                    : nullptr;
    // limits of the wave's first and last slot (rows only grow along the slots)
    const int64_t wlast = min(wbeg + 15, nslots - 1);
    const int wave_min_lim = wave_live ? clampi(causal_limit(seq, pre, r0), 0, W) : 0;
    const int wave_max_lim = wave_live ? clampi(causal_limit(seq, pre, (int)(wlast / a.H)), 0, W) : 0;
    // logits rows this lane writes out: slots wbeg + 2 q + wrow
    float* orow[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int k = 2 * q + wrow;
      const uint32_t hk = (uint32_t)h0 + (uint32_t)k;
      const int rk = r0 + (int)(hk / (uint32_t)a.H), hh = (int)(hk % (uint32_t)a.H);
      orow[q] = (wbeg + k < nslots)
                    ? a.lg + ((int64_t)row0 + rk) * a.lg_row_stride + (int64_t)hh * a.lg_head_stride
                    : nullptr;
    }

    const int j0 = pc * a.pages_per_item;
    const int j1 = min(j0 + a.pages_per_item, a.NB);
    const int jl = min(j1, (item_lim + P - 1) / P);   // pages [j0, jl) hold live tokens for some slot
    const int32_t* btrow = a.bt + (int64_t)b * a.bt_stride;

    // page ids, 64 at a time: lane l holds the id of page jid + l
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
      float* wcolp = win + i * kWinPitch + (j % PPW) * P + 4 * g;   // this lane's column of tile 0 in the window
      float m = kNegInf;
      bool scored = false;
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
        if (j * P < wave_max_lim) {   // some slot of this wave sees the page
          scored = true;
          const uint8_t* kb = kbuf + ((j - j0) & 1) * PB;
          const int lrel = lim - j * P - 4 * g;
          const bool mask = (j + 1) * P > wave_min_lim;
#pragma unroll
          for (int t = 0; t < TPP; ++t) {
            v4f c = mma_tile(lds_tile<KDT, P>(kb, g, i, t), qt);
            if (mask) {
#pragma unroll
              for (int v = 0; v < 4; ++v) c[v] = (16 * t + v < lrel) ? c[v] : kNegInf;
            }
            if constexpr (WANT_BS) m = max_into(m, c);
            *reinterpret_cast<v4f*>(wcolp + 16 * t) = c * s;
          }
        }
        if (more) stage_store<KDT, P>(nx, kbuf + ((j + 1 - j0) & 1) * PB, tid);
      }
      if (!scored) {
#pragma unroll
        for (int t = 0; t < TPP; ++t) *reinterpret_cast<v4f*>(wcolp + 16 * t) = ninf;
      }
      if constexpr (WANT_BS) {
        const float rr = fold_groups(m);
        if (g == 0 && bsp) bsp[j] = rr * s;
      }
      if ((j + 1) % PPW == 0 || j == j1 - 1) {
        // write out tokens [t0, tend) of the window; only this wave wrote its
        // window rows (a wave's LDS accesses complete in order; the fences
        // keep the compiler from moving these reads above those writes)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int wb = j - j % PPW;                    // first page of the window
        const int t0 = max(j0, wb) * P;                // first token written by this item
        const int tend = min((j + 1) * P, W);
        const int tok = wb * P + 4 * wcol;
        if (tok >= t0 && tok < tend) {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const v4f v = *reinterpret_cast<const v4f*>(win + (2 * q + wrow) * kWinPitch + 4 * wcol);
            if (orow[q]) store_logits4(orow[q], tok, v, tend, a.vec_lg);
          }
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
    const void* fn = a.bs ? reinterpret_cast<const void*>(&k_logits<QDT, KDT, P, true>)
                          : reinterpret_cast<const void*>(&k_logits<QDT, KDT, P, false>);
    return hipLaunchKernel(fn, dim3(plan.grid), dim3(kThreads), args, 0, stream);
  }
};

template <int QDT, int KDT, int P>
struct Occupancy {
  static int run(bool bs) { return bs ? occ_of(&k_logits<QDT, KDT, P, true>) : occ_of(&k_logits<QDT, KDT, P, false>); }
};

}  // namespace

hipError_t launch_logits(const mxs_plan& plan, const KArgs& a, hipStream_t stream) {
  return dispatch_variant<Launch>(plan.q_dtype, plan.k_dtype, plan.page_size, plan, a, stream);
}

int occupancy_logits(int32_t q_dtype, int32_t k_dtype, int32_t page_size, bool want_bs) {
  return dispatch_variant<Occupancy>(q_dtype, k_dtype, page_size, want_bs);
}

}  // namespace mxs
