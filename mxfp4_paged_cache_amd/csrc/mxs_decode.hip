// Decode kernel of the paged MXFP4 index scorer (gfx950).
#include "mxs_device.h"

namespace mxs {
namespace {
using namespace dev;

// ---------------------------------------------------------------------------
// Decode block scores: one wave per (request, group of 64 heads, chunk of <=
// 32 pages). (Decode calls that also want logits run on the logits kernel,
// one query row per request: its LDS windows write logit rows far faster
// than this kernel's MFMA layout would.)
// Each page is read by exactly one wave, so K goes straight from HBM into
// registers (staging it in LDS would buy nothing): per 16-token tile, lane
// (g, i) loads bytes 16g..16g+15 of token 16t+i (one 1 KB contiguous block
// per wave instruction) and e8m0 byte g of that token (an fp8 page takes a
// detour through LDS, see below). Pages are double-buffered in registers:
// the loads of page j+2 are in flight while page j+1 is scored. The chunk's page ids are read once into one VGPR (lane l holds
// the id of page j0 + l) and picked per page with readlane.
//
// Wave items are ordered page chunk fastest, and the plan makes the chunk
// count a multiple of 4, so the four waves of a workgroup share (request,
// head group): they load the query tiles once, one tile each, and exchange
// them through LDS. Workgroups are dispatched round-robin over the 8 XCDs;
// renumbering them so that each XCD gets a contiguous range of workgroups
// keeps all chunks of a request on one XCD, whose L2 then serves the
// request's query and block-table row to every chunk.
// ---------------------------------------------------------------------------
// One page in registers. load(): dr/sr are buffer resources over the page's
// data and scale bytes (uniform; empty for a refill past the chunk's last
// live page, whose loads then return zeros and move no bytes), doff/soff the
// lane's byte offsets inside the page (MXFP4: data 64 i + 16 g, scale
// 4 i + g; fp8: 16 * lane).
template <int KDT, int P>
struct RegPage;

template <int P>
struct RegPage<MXS_K_MXFP4, P> {
  static constexpr uint32_t kDataBytes = P * 64, kScaleBytes = P * 4;
  u4 d[P / 16];
  int s[P / 16];
  static __device__ __forceinline__ uint32_t data_offset(int g, int i) { return (uint32_t)(i * 64 + 16 * g); }
  __device__ __forceinline__ KTile<MXS_K_MXFP4> tile(int t) const { return {d[t], s[t]}; }
  __device__ __forceinline__ void load(rsrc_t dr, rsrc_t sr, uint32_t doff, uint32_t soff) {
#pragma unroll
    for (int t = 0; t < P / 16; ++t) {
      d[t] = buffer_load16_nt(dr, doff + 1024u * t);
      s[t] = buffer_load1_nt(sr, soff + 64u * t);
    }
  }
};

// fp8: a 16-token tile is 2 KB. Loaded as two contiguous 1 KB blocks (chunk
// `lane` and chunk 64 + `lane` of the tile), which the MFMA cannot take
// directly (its row i must sit in lanes i, i + 16, ...); each half page goes
// through the wave's LDS buffer in the fp8 tile layout and is read back per
// tile. Loading each token's slices straight into their MFMA lanes instead
// (16 pieces of 64 bytes per instruction) measured about 20% slower.
template <int P>
struct RegPage<MXS_K_E4M3, P> {
  static constexpr uint32_t kDataBytes = P * 128, kScaleBytes = 0;
  u4 c0[P / 16];   // chunk `lane` of tile t
  u4 c1[P / 16];   // chunk 64 + `lane` of tile t
  static __device__ __forceinline__ uint32_t data_offset(int g, int i) { return (uint32_t)(16 * (16 * g + i)); }
  __device__ __forceinline__ void load(rsrc_t dr, rsrc_t, uint32_t doff, uint32_t) {
#pragma unroll
    for (int t = 0; t < P / 16; ++t) {
      c0[t] = buffer_load16_nt(dr, doff + 2048u * t);
      c1[t] = buffer_load16_nt(dr, doff + 2048u * t + 1024u);
    }
  }
  // tiles [HF * P / 32, (HF + 1) * P / 32) into buf (P * 64 bytes) as tiles 0.. of the fp8 layout
  template <int HF>
  __device__ __forceinline__ void stage_half(uint8_t* buf, int lane) const {
#pragma unroll
    for (int u = 0; u < P / 32; ++u) {
      *reinterpret_cast<u4*>(buf + fp8_chunk_slot(u, lane)) = c0[HF * (P / 32) + u];
      *reinterpret_cast<u4*>(buf + fp8_chunk_slot(u, 64 + lane)) = c1[HF * (P / 32) + u];
    }
  }
};

// MFMAs and folds of tiles [T0, T1) of one page against the wave's four query
// tiles; tile(t) gives the K operand of tile t. MASK: the page holds the end
// of the live window (token 16 t + 4 g + v is live iff 16 t + v < lrel). The
// loop is software-pipelined by hand: the four MFMAs of tile t are issued
// before the results of tile t-1 are folded, and a scheduling fence after
// each step keeps only two tiles of results live.
template <int MASK, int T0, int T1, typename Tile>
__device__ __forceinline__ void decode_tiles(const Tile& tile, const v8i (&qt)[4], int lrel, float (&m)[4]) {
  v4f prev[4];
#pragma unroll
  for (int t = T0; t <= T1; ++t) {
    v4f cur[4];
    if (t < T1) {
#pragma unroll
      for (int n = 0; n < 4; ++n) cur[n] = mma_tile(tile(t), qt[n]);
    }
    if (t > T0) {
      const int tp = t - 1;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        v4f c = prev[n];
        if constexpr (MASK) {
#pragma unroll
          for (int v = 0; v < 4; ++v) c[v] = (16 * tp + v < lrel) ? c[v] : kNegInf;
        }
        m[n] = max_into(m[n], c);
      }
    }
    if (t < T1) {
#pragma unroll
      for (int n = 0; n < 4; ++n) prev[n] = cur[n];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Score one register-resident page (MASK: tokens >= lip are dead) and stage
// its block scores; kbuf is the wave's LDS buffer (fp8 only).
template <int KDT, int P, bool MASK>
__device__ __forceinline__ void decode_page(const RegPage<KDT, P>& kp, const v8i (&qt)[4], int lip, int g,
                                            float* stage, int jrel, const KArgs& a, uint8_t* kbuf) {
  constexpr int TPP = P / 16;
  float m[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  const int lrel = lip - 4 * g;
  if constexpr (KDT == MXS_K_MXFP4) {
    decode_tiles<MASK, 0, TPP>([&](int t) { return kp.tile(t); }, qt, lrel, m);
  } else {
    constexpr int HT = TPP / 2;
    const int lane = threadIdx.x & 63, i = lane & 15;
    auto from_lds = [&](int t0) { return [=](int t) { return lds_tile<MXS_K_E4M3, P>(kbuf, g, i, t - t0); }; };
    wave_lds_sync();   // the previous page's reads of kbuf are done
    kp.template stage_half<0>(kbuf, lane);
    wave_lds_sync();
    decode_tiles<MASK, 0, HT>(from_lds(0), qt, lrel, m);
    wave_lds_sync();
    kp.template stage_half<1>(kbuf, lane);
    wave_lds_sync();
    decode_tiles<MASK, HT, TPP>(from_lds(HT), qt, lrel, m);
  }
  const float s = a.sm_scale;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const float r = fold_groups(m[n]);
    if (g == 0) stage[(16 * n + (threadIdx.x & 15)) * kDecodeStageStride + jrel] = r * s;
  }
}

template <int QDT, int KDT, int P>
__global__ void __launch_bounds__(kThreads, 2) k_decode(KArgs a) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, i = lane & 15;
  // the wave index is uniform across the wave: keep everything derived from it scalar
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  int blk = blockIdx.x;
  if ((gridDim.x & 7) == 0) blk = (blk & 7) * (int)(gridDim.x >> 3) + (blk >> 3);
  // the plan launches exactly items / 4 workgroups; the guard only keeps a
  // stray wave harmless (it still takes part in the barrier below)
  const bool active = (int64_t)blk * kWaves + wave < a.items;
  const int64_t item = active ? (int64_t)blk * kWaves + wave : (int64_t)blk * kWaves;
  const int pc = (int)(item % a.page_items);
  const int64_t rest = item / a.page_items;
  const int hg = (int)(rest % a.head_groups);
  const int b = (int)(rest / a.head_groups);

  const int limit = clampi(a.seq[b], 0, a.max_seq_len);
  const int live_pages = (limit + P - 1) / P;
  const int j0 = pc * a.pages_per_item;
  const int j1 = max(j0, min(j0 + a.pages_per_item, a.NB));   // chunks past NB are empty
  const int jl = min(j1, live_pages);                 // pages [j0, jl) are scored

  // the chunk's page ids first (lane l: page j0 + l), so their latency overlaps the query loads
  const int my_page = (active && j0 + lane < jl) ? a.bt[(int64_t)b * a.bt_stride + j0 + lane] : 0;
  // query tile `wave` of the workgroup's 64 heads, rounded to e4m3, shared through LDS
  __shared__ v8i q_share[kWaves][64];
  {
    const int h = hg * kDecodeHeads + wave * 16 + i;
    const bool v = h < a.H;
    const int hc = v ? h : a.H - 1;
    q_share[wave][lane] =
        load_q_tile_masked<QDT>(a.q + (int64_t)b * a.q_row_stride + (int64_t)hc * a.q_head_stride, g, v);
  }
  __syncthreads();
  if (!active) return;
  v8i qt[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) qt[n] = q_share[n][lane];
  float* bs_row = a.bs + (int64_t)b * a.bs_row_stride;
  // this wave's staging area for its block scores: [64 heads][pages of the chunk]
  __shared__ float stage_all[kWaves][kDecodeHeads * kDecodeStageStride];
  float* stage = stage_all[wave];
  // fp8: this wave's half-page K buffer (P * 64 bytes)
  __shared__ __attribute__((aligned(16))) uint8_t kbuf_all[kWaves][KDT == MXS_K_E4M3 ? P * 64 : 16];
  uint8_t* kbuf = kbuf_all[wave];

  if (j0 < jl) {
    const uint32_t doff = RegPage<KDT, P>::data_offset(g, i);
    const uint32_t soff = (uint32_t)(i * 4 + g);
    // Refills past the chunk's last live page (the pipeline's tail) go
    // through empty buffer resources: they issue and retire like real loads,
    // so every wait stays exact, but fetch nothing (with the last live page
    // re-read instead, 34 page loads per 32-page chunk reached HBM).
    auto load_page = [&](RegPage<KDT, P>& kp, int j) {
      const bool live = j < jl;
      const int64_t page = __builtin_amdgcn_readlane(my_page, min(j, jl - 1) - j0);
      const rsrc_t dr = buffer_rsrc(a.kd + page * a.kd_page_stride, live ? RegPage<KDT, P>::kDataBytes : 0u);
      const rsrc_t sr = KDT == MXS_K_MXFP4
                            ? buffer_rsrc(a.ks + page * a.ks_page_stride, live ? RegPage<KDT, P>::kScaleBytes : 0u)
                            : dr;
      kp.load(dr, sr, doff, soff);
    };
    auto score = [&](const RegPage<KDT, P>& kp, int j) {
      const int lip = limit - j * P;                 // live tokens in this page
      if (lip >= P)
        decode_page<KDT, P, false>(kp, qt, lip, g, stage, j - j0, a, kbuf);
      else
        decode_page<KDT, P, true>(kp, qt, lip, g, stage, j - j0, a, kbuf);
    };
    RegPage<KDT, P> A, B;
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
  }
  // Block scores leave LDS as one contiguous run of (j1 - j0) floats per head:
  // consecutive lanes write consecutive pages, so every store instruction
  // covers whole cache lines instead of 64 scattered 4-byte words. The stores
  // are non-temporal (nothing here reads them back; 1% on the decode workload).
  const int npg = j1 - j0;
  const int nh = min(kDecodeHeads, a.H - hg * kDecodeHeads);
  for (int idx = lane; idx < nh * npg; idx += 64) {
    const int h = idx / npg, p = idx - h * npg;
    __builtin_nontemporal_store(stage[h * kDecodeStageStride + p],
                                bs_row + (int64_t)(hg * kDecodeHeads + h) * a.bs_head_stride + j0 + p);
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
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_decode<QDT, KDT, P>), dim3(plan.grid), dim3(kThreads),
                           args, 0, stream);
  }
};

template <int QDT, int KDT, int P>
struct Occupancy {
  static int run() { return occ_of(&k_decode<QDT, KDT, P>); }
};

}  // namespace

hipError_t launch_decode(const mxs_plan& plan, const KArgs& a, hipStream_t stream) {
  return dispatch_variant<Launch>(plan.q_dtype, plan.k_dtype, plan.page_size, plan, a, stream);
}

int occupancy_decode(int32_t q_dtype, int32_t k_dtype, int32_t page_size) {
  return dispatch_variant<Occupancy>(q_dtype, k_dtype, page_size);
}

}  // namespace mxs
