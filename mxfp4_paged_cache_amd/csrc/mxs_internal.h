// Internal interface between the host entry points (mxs_api.cpp) and the
// gfx950 kernels (mxs_decode.hip, mxs_prefill.hip, mxs_logits.hip,
// mxs_select.hip, mxs_write.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxscore.h"

namespace mxs {

// Kernel ids stored in mxs_plan::kernel.
enum KernelId : int32_t {
  KID_DECODE = 1,     // decode block scores: one wave per (request, head group, page chunk)
  KID_PREFILL = 2,    // block scores: workgroup per (request, 512 slots, page chunk); K staged in LDS
  KID_LOGITS = 3,     // logits (+ block scores), prefill or decode rows: workgroup per (request, 64 slots,
                      // page chunk); output via LDS windows
};

constexpr int kWaves = 4;           // waves per workgroup, every kernel
// Longest output window / context in tokens: page-rounded token indices
// (ceil(max_seq_len / P) * P) then stay within int32.
constexpr int32_t kMaxSeqLen = INT32_MAX - 255;
constexpr int kThreads = 64 * kWaves;
constexpr int kPrefillTiles = 8;    // 16-slot query tiles per wave (block-score kernel)
constexpr int kLogitsTiles = 1;     // 16-slot query tiles per wave (logits kernel)
constexpr int kDecodeHeads = 64;    // heads per decode wave (4 tiles of 16)
constexpr int kDecodeMaxPages = 32; // pages per decode wave (ids fit one VGPR; scores staged in LDS)
constexpr int kDecodeStageStride = kDecodeMaxPages + 1;   // LDS row pitch in floats (odd: no bank conflicts)

// Query slots per work item of the block-score and the logits kernel.
constexpr int kPrefillSlotsPerItem = kWaves * kPrefillTiles * 16;
constexpr int kLogitsSlotsPerItem = kWaves * kLogitsTiles * 16;

// Everything a kernel needs, by value. Byte strides for query and cache,
// element strides for int32 tables and fp32 outputs.
struct KArgs {
  const uint8_t* q;
  int64_t q_row_stride;     // bytes
  int64_t q_head_stride;    // bytes
  int32_t H;
  const uint8_t* kd;
  int64_t kd_page_stride;   // bytes
  const uint8_t* ks;        // e8m0 scales (MXFP4 cache; null for an fp8 cache)
  int64_t ks_page_stride;   // bytes
  const int32_t* bt;
  int64_t bt_stride;        // elements
  const int32_t* cu;        // prefill / logits
  const int32_t* seq;
  const int32_t* prefix;    // prefill / logits
  int32_t B;
  int32_t max_seq_len;
  int32_t NB;
  float sm_scale;
  float* bs;                // block scores (may be null in logits mode)
  int64_t bs_row_stride;
  int64_t bs_head_stride;
  float* lg;                // logits (may be null in prefill / decode)
  int64_t lg_row_stride;
  int64_t lg_head_stride;
  int32_t slots_per_item;
  int32_t pages_per_item;
  int32_t slot_items;
  int32_t page_items;
  int32_t head_groups;
  int64_t items;
  int32_t vec_bs;           // widest vector store the block-score rows allow, in floats (4, 2 or 1)
  int32_t vec_lg;           // logit rows 16-byte aligned
  int32_t decode_rows;      // logits kernel: row b is request b (one query row, limit = seq_len[b])
  int32_t xcd_split;        // logits kernel: XCD x takes items [x * items / 8, (x + 1) * items / 8)
};

// Arguments of the page-selection kernel (mxs_select.hip).
struct SArgs {
  const float* bs;          // block scores [rows, H, NB]
  int64_t bs_row_stride;    // elements
  int64_t bs_head_stride;
  int32_t* out;             // selected pages [rows, H, k]
  int64_t out_row_stride;   // elements
  int64_t out_head_stride;
  const int32_t* cu;        // prefill rows: cu_seqlens_q, seq_lens, prefix_lens
  const int32_t* seq;
  const int32_t* prefix;
  int32_t decode;           // 1: row b is request b, its limit is seq_lens[b]
  int32_t B;
  int32_t H;
  int32_t NB;
  int32_t P;
  int32_t k;
  int32_t max_seq_len;
  int64_t items;            // rows * H
};
constexpr int kSelectMaxPages = 64 * 64;   // scores per (row, head) the selection kernel holds (64 per lane)

// Arguments of the writer kernel (mxs_write.hip).
struct WArgs {
  const uint16_t* k;        // bf16 keys [n, 128]
  int64_t k_row_stride;     // elements
  const int64_t* slots;     // [n]: page * P + offset, or -1
  int64_t n;
  uint8_t* kd;
  int64_t kd_page_stride;   // bytes
  uint8_t* ks;              // MXFP4 only
  int64_t ks_page_stride;   // bytes
  int64_t num_pages;
  int32_t P;
  int32_t kdt;              // MXS_K_MXFP4 or MXS_K_E4M3
};

// Arguments of the attention-decode kernel (mxs_attn.hip).
struct AArgs {
  const uint8_t* q;
  int64_t q_row_stride;     // bytes
  int64_t q_head_stride;    // bytes
  const uint8_t* kd;
  int64_t kd_page_stride, kd_head_stride;   // bytes
  const uint8_t* ks;
  int64_t ks_page_stride, ks_head_stride;
  const uint8_t* vd;
  int64_t vd_page_stride, vd_head_stride;
  const uint8_t* vs;
  int64_t vs_page_stride, vs_head_stride;
  const int32_t* bt;
  int64_t bt_stride;        // elements
  const int32_t* ctx;
  int32_t R;                // rows
  int32_t Hkv;
  int32_t G;                // query heads per kv head, 1..16
  int32_t max_context;
  float scale_log2e;        // scale * log2(e): the softmax runs in exp2
  uint16_t* out;            // bf16
  int64_t out_row_stride;   // elements
  int64_t out_head_stride;
};

// Launchers. Return the HIP status of the launch.
hipError_t launch_attn(int32_t q_dtype, int32_t page_size, const AArgs& a, hipStream_t stream);
hipError_t launch_select(int per, int64_t grid, const SArgs& a, hipStream_t stream);
hipError_t launch_write(int64_t grid, const WArgs& a, hipStream_t stream);
hipError_t launch_decode(const mxs_plan& plan, const KArgs& a, hipStream_t stream);
hipError_t launch_prefill(const mxs_plan& plan, const KArgs& a, hipStream_t stream);
hipError_t launch_logits(const mxs_plan& plan, const KArgs& a, hipStream_t stream);

// Workgroups of the kernel variant (q dtype, cache dtype, page size, outputs) that fit on one CU.
int occupancy_decode(int32_t q_dtype, int32_t k_dtype, int32_t page_size);
int occupancy_prefill(int32_t q_dtype, int32_t k_dtype, int32_t page_size);
int occupancy_logits(int32_t q_dtype, int32_t k_dtype, int32_t page_size, bool want_bs);

inline hipError_t launch(const mxs_plan& plan, const KArgs& a, hipStream_t stream) {
  return plan.kernel == KID_DECODE    ? launch_decode(plan, a, stream)
         : plan.kernel == KID_PREFILL ? launch_prefill(plan, a, stream)
                                      : launch_logits(plan, a, stream);
}

inline int occupancy(int32_t kernel, int32_t q_dtype, int32_t k_dtype, int32_t page_size, bool want_bs, bool want_lg) {
  return kernel == KID_DECODE    ? occupancy_decode(q_dtype, k_dtype, page_size)
         : kernel == KID_PREFILL ? occupancy_prefill(q_dtype, k_dtype, page_size)
                                 : occupancy_logits(q_dtype, k_dtype, page_size, want_bs);
}

// F<QDT, KDT, P>::run(args...) for one (query dtype, cache dtype, page size).
template <template <int, int, int> class F, typename... Args>
inline auto dispatch_variant(int32_t q_dtype, int32_t k_dtype, int32_t page_size, Args&&... args) {
  if (q_dtype == MXS_Q_BF16) {
    if (k_dtype == MXS_K_E4M3)
      return page_size == 128 ? F<MXS_Q_BF16, MXS_K_E4M3, 128>::run(args...) : F<MXS_Q_BF16, MXS_K_E4M3, 64>::run(args...);
    return page_size == 128 ? F<MXS_Q_BF16, MXS_K_MXFP4, 128>::run(args...) : F<MXS_Q_BF16, MXS_K_MXFP4, 64>::run(args...);
  }
  if (k_dtype == MXS_K_E4M3)
    return page_size == 128 ? F<MXS_Q_E4M3, MXS_K_E4M3, 128>::run(args...) : F<MXS_Q_E4M3, MXS_K_E4M3, 64>::run(args...);
  return page_size == 128 ? F<MXS_Q_E4M3, MXS_K_MXFP4, 128>::run(args...) : F<MXS_Q_E4M3, MXS_K_MXFP4, 64>::run(args...);
}

}  // namespace mxs
