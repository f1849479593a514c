// Host side of the C ABI declared in include/mxscore.h: argument validation,
// launch planning and dispatch. Everything here runs before any device work;
// a rejected call touches no memory (aiter #7061, "Changed op tests":
// rejections are raised before launch).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <algorithm>
#include <mutex>
#include <vector>
#include <string>

#include "mxs_internal.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// a * b + c without overflow; returns false on overflow or negative inputs
bool mul_add(int64_t a, int64_t b, int64_t c, int64_t* out) {
  if (a < 0 || b < 0 || c < 0) return false;
  __int128 r = (__int128)a * b + c;
  if (r > INT64_MAX) return false;
  *out = (int64_t)r;
  return true;
}

struct DeviceInfo {
  int status = MXS_OK;
  std::string why;
  int cus = 0;
};

std::mutex g_mu;
std::map<int, DeviceInfo> g_devices;
std::map<uint64_t, int> g_occupancy;

int current_device(int* dev, DeviceInfo* info) {
  int d = -1;
  if (hipGetDevice(&d) != hipSuccess || d < 0) {
    (void)hipGetLastError();
    return fail(MXS_EUNSUPPORTED, "no HIP device is available");
  }
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_devices.find(d);
  if (it == g_devices.end()) {
    DeviceInfo di;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, d) != hipSuccess) {
      (void)hipGetLastError();
      di.status = MXS_EUNSUPPORTED;
      di.why = "cannot query the current HIP device";
    } else if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      di.status = MXS_EUNSUPPORTED;
      di.why = std::string("the scorer needs gfx950 (MI355X); current device is ") + prop.gcnArchName;
    } else {
      di.cus = prop.multiProcessorCount;
    }
    it = g_devices.emplace(d, di).first;
  }
  *dev = d;
  *info = it->second;
  if (info->status != MXS_OK) return fail(info->status, "%s", info->why.c_str());
  return MXS_OK;
}

int occupancy_cached(int dev, int32_t kernel, int32_t q_dtype, int32_t k_dtype, int32_t page_size, bool want_bs,
                     bool want_lg) {
  const uint64_t key = ((uint64_t)(uint32_t)dev << 32) | ((uint64_t)kernel << 16) | ((uint64_t)q_dtype << 8) |
                       (uint64_t)(page_size == 128 ? 1 : 0) | (want_bs ? 2u : 0u) | (want_lg ? 4u : 0u) |
                       (k_dtype == MXS_K_E4M3 ? 8u : 0u);
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_occupancy.find(key);
    if (it != g_occupancy.end()) return it->second;
  }
  const int occ = mxs::occupancy(kernel, q_dtype, k_dtype, page_size, want_bs, want_lg);
  std::lock_guard<std::mutex> lock(g_mu);
  g_occupancy[key] = occ;
  return occ;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int check_k_dtype(int32_t k_dtype) {
  if (k_dtype != MXS_K_MXFP4 && k_dtype != MXS_K_E4M3)
    return fail(MXS_EDTYPE, "cache dtype must be MXFP4 (%d) or e4m3 (%d); got %d", MXS_K_MXFP4, MXS_K_E4M3, k_dtype);
  return MXS_OK;
}

// The cache views of either format (page size and dtype already checked):
// MXFP4 needs both views, an fp8 cache only the data view (128 B a token).
int check_kcache_views(const mxs_kcache* k) {
  const int P = k->page_size;
  const bool fp8 = k->k_dtype == MXS_K_E4M3;
  const int64_t token_bytes = fp8 ? 128 : 64;
  if (!k->data || (!fp8 && !k->scale)) return fail(MXS_EINVAL, "cache data and scale pointers must not be NULL");
  if (!aligned(k->data, 16)) return fail(MXS_ELAYOUT, "cache data view must be 16-byte aligned");
  if (!fp8 && !aligned(k->scale, 4)) return fail(MXS_ELAYOUT, "cache scale view must be 4-byte aligned");
  if (k->data_page_stride < (int64_t)P * token_bytes || k->data_page_stride % 16)
    return fail(MXS_ELAYOUT, "data page stride %lld must be a multiple of 16 and >= %lld (narrow data view)",
                (long long)k->data_page_stride, (long long)(P * token_bytes));
  if (!fp8 && (k->scale_page_stride < (int64_t)P * 4 || k->scale_page_stride % 4))
    return fail(MXS_ELAYOUT, "scale page stride %lld must be a multiple of 4 and >= %d (narrow scale view)",
                (long long)k->scale_page_stride, P * 4);
  if (k->num_pages < 1) return fail(MXS_EINVAL, "num_pages must be >= 1");
  int64_t tmp;
  if (!mul_add(k->num_pages, k->data_page_stride, 0, &tmp) ||
      (!fp8 && !mul_add(k->num_pages, k->scale_page_stride, 0, &tmp)))
    return fail(MXS_ELAYOUT, "cache span overflows 64 bits");
  return MXS_OK;
}

}  // namespace

extern "C" {

const char* mxs_last_error(void) { return g_error.c_str(); }

int mxs_write_pages(const void* k, int64_t k_row_stride, int64_t num_tokens, const int64_t* slot_mapping,
                    const mxs_kcache* c, void* stream) {
  if (!c) return fail(MXS_EINVAL, "cache descriptor must not be NULL");
  if (num_tokens < 0) return fail(MXS_EINVAL, "num_tokens must be >= 0");
  if (c->page_size != 64 && c->page_size != 128)
    return fail(MXS_ELAYOUT, "page_size must be 64 or 128, got %d", c->page_size);
  if (check_k_dtype(c->k_dtype)) return MXS_EDTYPE;
  if (num_tokens == 0) return MXS_OK;
  if (!k || !slot_mapping) return fail(MXS_EINVAL, "keys and slot_mapping must not be NULL");
  if (!aligned(k, 16) || k_row_stride < 128 || k_row_stride % 8)
    return fail(MXS_ELAYOUT, "key rows must be 16-byte aligned with a row stride >= 128 elements");
  if (!aligned(slot_mapping, 8)) return fail(MXS_ELAYOUT, "slot_mapping must be 8-byte aligned");
  const int P = c->page_size;
  int rc0 = check_kcache_views(c);
  if (rc0 != MXS_OK) return rc0;
  int64_t tmp;
  if (!mul_add(num_tokens, k_row_stride, 0, &tmp)) return fail(MXS_ELAYOUT, "span overflows 64 bits");
  int dev;
  DeviceInfo info;
  int rc = current_device(&dev, &info);
  if (rc != MXS_OK) return rc;
  mxs::WArgs a;
  std::memset(&a, 0, sizeof a);
  a.k = static_cast<const uint16_t*>(k);
  a.k_row_stride = k_row_stride;
  a.slots = slot_mapping;
  a.n = num_tokens;
  a.kd = static_cast<uint8_t*>(const_cast<void*>(c->data));
  a.kd_page_stride = c->data_page_stride;
  a.ks = c->k_dtype == MXS_K_E4M3 ? nullptr : static_cast<uint8_t*>(const_cast<void*>(c->scale));
  a.ks_page_stride = c->scale_page_stride;
  a.num_pages = c->num_pages;
  a.P = P;
  a.kdt = c->k_dtype;
  const int64_t waves = ceil_div(ceil_div(num_tokens, 4), 4);   // 4 steps of 4 tokens per wave
  const int64_t grid = std::min<int64_t>(ceil_div(waves, mxs::kWaves), (int64_t)info.cus * 16);
  if (mxs::launch_write(grid, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(MXS_EDEVICE, "launching the writer failed: %s", hipGetErrorString(hipGetLastError()));
  return MXS_OK;
}

int mxs_select_pages(int32_t mode, const mxs_batch* bt, int32_t num_heads, int32_t page_size,
                     const float* block_scores, int64_t bs_row_stride, int64_t bs_head_stride, int32_t k,
                     int32_t* pages, int64_t pages_row_stride, int64_t pages_head_stride, void* stream) {
  if (!bt) return fail(MXS_EINVAL, "batch descriptor must not be NULL");
  if (mode != MXS_MODE_PREFILL && mode != MXS_MODE_DECODE && mode != MXS_MODE_LOGITS)
    return fail(MXS_EINVAL, "unknown mode %d", mode);
  if (page_size != 64 && page_size != 128) return fail(MXS_ELAYOUT, "page_size must be 64 or 128, got %d", page_size);
  if (num_heads < 1) return fail(MXS_EINVAL, "num_heads must be >= 1, got %d", num_heads);
  if (k < 0) return fail(MXS_EINVAL, "k must be >= 0, got %d", k);
  if (bt->batch < 0 || bt->max_seq_len < 0) return fail(MXS_EINVAL, "batch and max_seq_len must be >= 0");
  if (bt->max_seq_len > mxs::kMaxSeqLen)
    return fail(MXS_EINVAL, "max_seq_len %d is above the limit %d", bt->max_seq_len, mxs::kMaxSeqLen);
  const bool decode = mode == MXS_MODE_DECODE;
  if (!decode && bt->total_rows < 0) return fail(MXS_EINVAL, "total_rows must be >= 0");
  const int64_t rows = decode ? bt->batch : bt->total_rows;
  const int64_t NB = ceil_div(bt->max_seq_len, page_size);
  if (k == 0 || rows == 0 || bt->batch == 0) return MXS_OK;
  if (NB > mxs::kSelectMaxPages)
    return fail(MXS_EUNSUPPORTED, "selection holds at most %d pages per row, got %lld", mxs::kSelectMaxPages,
                (long long)NB);
  // an empty window (NB = 0) reads no score, and its score tensor may be empty (NULL)
  if ((!block_scores && NB > 0) || !pages) return fail(MXS_EINVAL, "block_scores and pages must not be NULL");
  if (!aligned(block_scores, 4) || !aligned(pages, 4)) return fail(MXS_ELAYOUT, "buffers must be 4-byte aligned");
  if (!bt->seq_lens || (!decode && (!bt->cu_seqlens_q || !bt->prefix_lens)))
    return fail(MXS_EINVAL, "seq_lens (and for prefill cu_seqlens_q, prefix_lens) must not be NULL");
  auto check_view = [&](const char* name, int64_t rs, int64_t hs, int64_t width) {
    if (rs < 0 || hs < 0) return fail(MXS_ELAYOUT, "%s strides must be >= 0", name);
    if (num_heads > 1 && hs < width) return fail(MXS_ELAYOUT, "%s head stride is narrower than its width", name);
    int64_t row_span, span;
    if (!mul_add(num_heads - 1, hs, width, &row_span)) return fail(MXS_ELAYOUT, "%s span overflows", name);
    if (rows > 1 && rs < row_span) return fail(MXS_ELAYOUT, "%s row stride is narrower than one row", name);
    if (!mul_add(rows - 1, rs, row_span, &span) || span > INT64_MAX / 4)
      return fail(MXS_ELAYOUT, "%s span overflows", name);
    return MXS_OK;
  };
  int rc = check_view("block_scores", bs_row_stride, bs_head_stride, NB);
  if (rc) return rc;
  rc = check_view("pages", pages_row_stride, pages_head_stride, k);
  if (rc) return rc;
  int dev;
  DeviceInfo info;
  rc = current_device(&dev, &info);
  if (rc != MXS_OK) return rc;
  mxs::SArgs a;
  std::memset(&a, 0, sizeof a);
  a.bs = block_scores;
  a.bs_row_stride = bs_row_stride;
  a.bs_head_stride = bs_head_stride;
  a.out = pages;
  a.out_row_stride = pages_row_stride;
  a.out_head_stride = pages_head_stride;
  a.cu = decode ? nullptr : bt->cu_seqlens_q;
  a.seq = bt->seq_lens;
  a.prefix = decode ? nullptr : bt->prefix_lens;
  a.decode = decode ? 1 : 0;
  a.B = bt->batch;
  a.H = num_heads;
  a.NB = (int32_t)NB;
  a.P = page_size;
  a.k = k;
  a.max_seq_len = bt->max_seq_len;
  a.items = rows * num_heads;
  const int per = (int)ceil_div(NB > 0 ? NB : 1, 64);
  // one wave per (row, head) while that fills the chip a few times over; beyond, waves loop
  const int64_t cap = (int64_t)info.cus * 32;
  const int64_t grid = std::min<int64_t>(ceil_div(a.items, mxs::kWaves), cap);
  if (mxs::launch_select(per, grid, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(MXS_EDEVICE, "launching the page selection failed: %s", hipGetErrorString(hipGetLastError()));
  return MXS_OK;
}

int mxs_check_metadata(int32_t mode, const mxs_kcache* k, const mxs_batch* bt, int32_t check_scales, void* stream) {
  if (!k || !bt) return fail(MXS_EINVAL, "cache and batch descriptors must not be NULL");
  if (mode != MXS_MODE_PREFILL && mode != MXS_MODE_DECODE && mode != MXS_MODE_LOGITS)
    return fail(MXS_EINVAL, "unknown mode %d", mode);
  if (k->page_size != 64 && k->page_size != 128)
    return fail(MXS_ELAYOUT, "page_size must be 64 or 128, got %d", k->page_size);
  if (check_k_dtype(k->k_dtype)) return MXS_EDTYPE;
  const bool decode = mode == MXS_MODE_DECODE;
  const bool fp8 = k->k_dtype == MXS_K_E4M3;
  const int32_t B = bt->batch, P = k->page_size;
  if (B < 0 || bt->max_seq_len < 0) return fail(MXS_EINVAL, "batch and max_seq_len must be >= 0");
  if (bt->max_seq_len > mxs::kMaxSeqLen)
    return fail(MXS_EINVAL, "max_seq_len %d is above the limit %d", bt->max_seq_len, mxs::kMaxSeqLen);
  if (B == 0) return MXS_OK;
  if (!bt->block_table || !bt->seq_lens || (!decode && (!bt->cu_seqlens_q || !bt->prefix_lens)))
    return fail(MXS_EINVAL, "metadata pointers must not be NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto copy = [&](void* dst, const void* src, size_t n) {
    return hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToHost, st) == hipSuccess;
  };
  std::vector<int32_t> seq(B), cu(decode ? 0 : B + 1), pre(decode ? 0 : B);
  if (!copy(seq.data(), bt->seq_lens, 4 * (size_t)B) ||
      (!decode && (!copy(cu.data(), bt->cu_seqlens_q, 4 * (size_t)(B + 1)) ||
                   !copy(pre.data(), bt->prefix_lens, 4 * (size_t)B))) ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(MXS_EDEVICE, "copying the request metadata failed");
  if (!decode) {
    if (cu[0] != 0) return fail(MXS_EINVAL, "cu_seqlens_q[0] is %d, not 0", cu[0]);
    for (int32_t b = 0; b < B; ++b) {
      const int64_t ql = (int64_t)cu[b + 1] - cu[b];
      if (ql < 0) return fail(MXS_EINVAL, "cu_seqlens_q decreases at request %d", b);
      if (ql > bt->max_query_len)
        return fail(MXS_EINVAL, "request %d has %lld query rows, more than max_query_len %d", b, (long long)ql,
                    bt->max_query_len);
      if (pre[b] < 0) return fail(MXS_EINVAL, "prefix_lens[%d] is negative (%d)", b, pre[b]);
    }
    if (cu[B] != bt->total_rows)
      return fail(MXS_EINVAL, "cu_seqlens_q[batch] is %d, total_rows is %d", cu[B], bt->total_rows);
  }
  // live tokens of each request: the largest limit over its rows
  std::vector<int64_t> live(B);
  for (int32_t b = 0; b < B; ++b) {
    if (seq[b] < 0 || seq[b] > bt->max_seq_len)
      return fail(MXS_EINVAL, "seq_lens[%d] is %d, outside [0, max_seq_len = %d]", b, seq[b], bt->max_seq_len);
    int64_t lim = seq[b];
    if (!decode) {
      const int64_t ql = (int64_t)cu[b + 1] - cu[b];
      lim = ql > 0 ? std::min<int64_t>(seq[b], (int64_t)pre[b] + ql) : 0;
    }
    live[b] = lim;
  }
  std::vector<int32_t> row;
  std::vector<uint8_t> sc;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t pages = ceil_div(live[b], P);
    if (pages == 0) continue;
    if (pages > bt->bt_width)
      return fail(MXS_EINVAL, "request %d has %lld live pages, more than the block table width %d", b,
                  (long long)pages, bt->bt_width);
    row.resize(pages);
    if (!copy(row.data(), bt->block_table + (int64_t)b * bt->bt_row_stride, 4 * (size_t)pages) ||
        hipStreamSynchronize(st) != hipSuccess)
      return fail(MXS_EDEVICE, "copying block-table row %d failed", b);
    for (int64_t j = 0; j < pages; ++j)
      if (row[j] < 0 || row[j] >= k->num_pages)
        return fail(MXS_EINVAL, "block_table[%d][%lld] = %d is outside [0, num_pages = %lld) for a live page", b,
                    (long long)j, row[j], (long long)k->num_pages);
    if (!check_scales) continue;
    if (fp8) {
      // live tokens of an fp8 cache must hold no NaN byte
      sc.resize((size_t)P * 128);
      for (int64_t j = 0; j < pages; ++j) {
        if (!copy(sc.data(), static_cast<const uint8_t*>(k->data) + (int64_t)row[j] * k->data_page_stride, sc.size()) ||
            hipStreamSynchronize(st) != hipSuccess)
          return fail(MXS_EDEVICE, "copying the data of page %d failed", row[j]);
        const int64_t ntok = std::min<int64_t>(P, live[b] - j * P);
        for (int64_t t = 0; t < ntok * 128; ++t)
          if ((sc[t] & 0x7F) == 0x7F)
            return fail(MXS_EINVAL, "request %d, token %lld: e4m3 byte 0x%02X is NaN", b, (long long)(j * P + t / 128),
                        sc[t]);
      }
      continue;
    }
    sc.resize((size_t)P * 4);
    for (int64_t j = 0; j < pages; ++j) {
      if (!copy(sc.data(), static_cast<const uint8_t*>(k->scale) + (int64_t)row[j] * k->scale_page_stride, sc.size()) ||
          hipStreamSynchronize(st) != hipSuccess)
        return fail(MXS_EDEVICE, "copying the scales of page %d failed", row[j]);
      const int64_t ntok = std::min<int64_t>(P, live[b] - j * P);
      for (int64_t t = 0; t < ntok * 4; ++t)
        if (sc[t] == 0 || sc[t] == 255)
          return fail(MXS_EINVAL, "request %d, token %lld: e8m0 byte %d outside [1, 254]", b,
                      (long long)(j * P + t / 4), sc[t]);
    }
  }
  return MXS_OK;
}

const char* mxs_version(void) { return "mxscore 0.1 (gfx950)"; }

int mxs_attn_decode(const mxs_query* q, const mxs_kvcache* kv, const int32_t* block_table, int64_t bt_row_stride,
                    int32_t bt_width, const int32_t* context_lens, int32_t num_rows, int32_t max_context, float scale,
                    void* out, int64_t out_row_stride, int64_t out_head_stride, void* stream) {
  if (!q || !kv) return fail(MXS_EINVAL, "query and cache descriptors must not be NULL");
  if (q->dtype != MXS_Q_BF16 && q->dtype != MXS_Q_E4M3)
    return fail(MXS_EDTYPE, "query dtype must be bf16 (%d) or e4m3 (%d); got %d", MXS_Q_BF16, MXS_Q_E4M3, q->dtype);
  if (kv->page_size != 64 && kv->page_size != 128)
    return fail(MXS_ELAYOUT, "page_size must be 64 or 128, got %d", kv->page_size);
  if (kv->num_kv_heads < 1 || q->num_heads < 1 || q->num_heads % kv->num_kv_heads)
    return fail(MXS_EINVAL, "query heads (%d) must be a positive multiple of kv heads (%d)", q->num_heads,
                kv->num_kv_heads);
  const int32_t G = q->num_heads / kv->num_kv_heads;
  if (G > 16) return fail(MXS_EUNSUPPORTED, "at most 16 query heads per kv head, got %d", G);
  if (num_rows < 0 || max_context < 0) return fail(MXS_EINVAL, "num_rows and max_context must be >= 0");
  if (max_context > mxs::kMaxSeqLen)
    return fail(MXS_EINVAL, "max_context %d is above the limit %d", max_context, mxs::kMaxSeqLen);
  if (!(std::isfinite(scale) && scale > 0.0f)) return fail(MXS_EINVAL, "scale must be finite and > 0");
  if (num_rows == 0) return MXS_OK;
  const int P = kv->page_size, Hkv = kv->num_kv_heads;
  // query
  const int64_t es = q->dtype == MXS_Q_BF16 ? 2 : 1;
  if (!q->ptr) return fail(MXS_EINVAL, "query pointer is NULL");
  if (!aligned(q->ptr, 16) || q->row_stride < 0 || q->head_stride < 0 || (q->row_stride * es) % 16 ||
      (q->head_stride * es) % 16)
    return fail(MXS_ELAYOUT, "query rows must be 16-byte aligned with strides in multiples of 16 bytes");
  // cache views
  auto check_view = [&](const char* name, const mxs_kvview& v) {
    if (!v.data || !v.scale) return fail(MXS_EINVAL, "%s data and scale pointers must not be NULL", name);
    if (!aligned(v.data, 16) || !aligned(v.scale, 4)) return fail(MXS_ELAYOUT, "%s views misaligned", name);
    if (v.data_head_stride % 16 || v.data_page_stride % 16 || v.scale_head_stride % 4 || v.scale_page_stride % 4 ||
        v.data_head_stride < 0 || v.scale_head_stride < 0)
      return fail(MXS_ELAYOUT, "%s strides must be multiples of 16 (data) and 4 (scale) bytes", name);
    if (Hkv > 1 && (v.data_head_stride < (int64_t)P * 64 || v.scale_head_stride < (int64_t)P * 4))
      return fail(MXS_ELAYOUT, "%s head strides are narrower than a page of one head", name);
    int64_t dspan, sspan;
    if (!mul_add(Hkv - 1, v.data_head_stride, (int64_t)P * 64, &dspan) ||
        !mul_add(Hkv - 1, v.scale_head_stride, (int64_t)P * 4, &sspan))
      return fail(MXS_ELAYOUT, "%s span overflows", name);
    if (kv->num_pages > 1 && (v.data_page_stride < dspan || v.scale_page_stride < sspan))
      return fail(MXS_ELAYOUT, "%s page strides are narrower than a page of all kv heads", name);
    int64_t tmp;
    if (!mul_add(kv->num_pages, v.data_page_stride, dspan, &tmp) || !mul_add(kv->num_pages, v.scale_page_stride, sspan, &tmp))
      return fail(MXS_ELAYOUT, "%s span overflows 64 bits", name);
    return MXS_OK;
  };
  if (kv->num_pages < 1) return fail(MXS_EINVAL, "num_pages must be >= 1");
  int rc = check_view("K", kv->k);
  if (rc) return rc;
  rc = check_view("V", kv->v);
  if (rc) return rc;
  // metadata and output
  if (!block_table || !context_lens) return fail(MXS_EINVAL, "block_table and context_lens must not be NULL");
  if (!aligned(block_table, 4) || !aligned(context_lens, 4)) return fail(MXS_ELAYOUT, "int32 metadata misaligned");
  if (bt_width < ceil_div(max_context, P))
    return fail(MXS_ELAYOUT, "block table width %d is narrower than ceil(max_context / page_size) = %lld", bt_width,
                (long long)ceil_div(max_context, P));
  if (num_rows > 1 && bt_row_stride < bt_width) return fail(MXS_ELAYOUT, "block table row stride below its width");
  if (!out) return fail(MXS_EINVAL, "output pointer is NULL");
  if (!aligned(out, 2) || out_row_stride < 0 || out_head_stride < 0)
    return fail(MXS_ELAYOUT, "output must be 2-byte aligned with strides >= 0");
  if (q->num_heads > 1 && out_head_stride < 128) return fail(MXS_ELAYOUT, "output head stride below 128 elements");
  int64_t row_span;
  if (!mul_add(q->num_heads - 1, out_head_stride, 128, &row_span) || (num_rows > 1 && out_row_stride < row_span))
    return fail(MXS_ELAYOUT, "output row stride below one row");
  if ((int64_t)num_rows * Hkv > INT32_MAX) return fail(MXS_EINVAL, "problem too large");
  int dev;
  DeviceInfo info;
  rc = current_device(&dev, &info);
  if (rc != MXS_OK) return rc;
  mxs::AArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = static_cast<const uint8_t*>(q->ptr);
  a.q_row_stride = q->row_stride * es;
  a.q_head_stride = q->head_stride * es;
  a.kd = static_cast<const uint8_t*>(kv->k.data);
  a.kd_page_stride = kv->k.data_page_stride;
  a.kd_head_stride = kv->k.data_head_stride;
  a.ks = static_cast<const uint8_t*>(kv->k.scale);
  a.ks_page_stride = kv->k.scale_page_stride;
  a.ks_head_stride = kv->k.scale_head_stride;
  a.vd = static_cast<const uint8_t*>(kv->v.data);
  a.vd_page_stride = kv->v.data_page_stride;
  a.vd_head_stride = kv->v.data_head_stride;
  a.vs = static_cast<const uint8_t*>(kv->v.scale);
  a.vs_page_stride = kv->v.scale_page_stride;
  a.vs_head_stride = kv->v.scale_head_stride;
  a.bt = block_table;
  a.bt_stride = bt_row_stride;
  a.ctx = context_lens;
  a.R = num_rows;
  a.Hkv = Hkv;
  a.G = G;
  a.max_context = max_context;
  a.scale_log2e = (float)((double)scale * 1.4426950408889634);
  a.out = static_cast<uint16_t*>(out);
  a.out_row_stride = out_row_stride;
  a.out_head_stride = out_head_stride;
  if (mxs::launch_attn(q->dtype, P, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(MXS_EDEVICE, "launching the attention decode failed: %s", hipGetErrorString(hipGetLastError()));
  return MXS_OK;
}

// Pure planner: every input is a host integer; the same inputs give the same
// plan. num_cus and wg_per_cu describe the device (CUs and resident
// workgroups of the chosen kernel per CU).
int mxs_plan_make_for(int32_t mode, int32_t q_dtype, int32_t k_dtype, int32_t page_size, int32_t num_heads,
                      int32_t batch, int32_t max_query_len, int32_t max_seq_len, int32_t want_logits,
                      int32_t want_blocks, int32_t parallel_unit_num, int32_t num_cus, int32_t wg_per_cu,
                      mxs_plan* plan) {
  if (!plan) return fail(MXS_EINVAL, "plan pointer is NULL");
  if (mode != MXS_MODE_PREFILL && mode != MXS_MODE_DECODE && mode != MXS_MODE_LOGITS)
    return fail(MXS_EINVAL, "unknown mode %d", mode);
  if (q_dtype != MXS_Q_BF16 && q_dtype != MXS_Q_E4M3)
    return fail(MXS_EDTYPE, "query dtype must be bf16 (%d) or e4m3 (%d); got %d (fp16 is refused)", MXS_Q_BF16,
                MXS_Q_E4M3, q_dtype);
  if (check_k_dtype(k_dtype)) return MXS_EDTYPE;
  if (page_size != 64 && page_size != 128) return fail(MXS_ELAYOUT, "page_size must be 64 or 128, got %d", page_size);
  if (num_heads < 1) return fail(MXS_EINVAL, "num_heads must be >= 1, got %d", num_heads);
  if (batch < 0 || max_seq_len < 0 || (mode != MXS_MODE_DECODE && max_query_len < 0))
    return fail(MXS_EINVAL, "negative batch (%d), max_query_len (%d) or max_seq_len (%d)", batch, max_query_len,
                max_seq_len);
  if (max_seq_len > mxs::kMaxSeqLen)
    return fail(MXS_EINVAL, "max_seq_len %d is above the limit %d", max_seq_len, mxs::kMaxSeqLen);
  if (parallel_unit_num < 0) return fail(MXS_EINVAL, "parallel_unit_num must be >= 0");
  if (num_cus < 1 || wg_per_cu < 1) return fail(MXS_EINVAL, "device description must be positive");
  if (mode == MXS_MODE_LOGITS && !want_logits) return fail(MXS_EINVAL, "logits mode needs logits");
  if (mode != MXS_MODE_LOGITS && !want_blocks) return fail(MXS_EINVAL, "prefill and decode need block scores");

  mxs_plan p;
  std::memset(&p, 0, sizeof p);
  p.mode = mode;
  p.q_dtype = q_dtype;
  p.k_dtype = k_dtype;
  p.page_size = page_size;
  p.num_heads = num_heads;
  p.batch = batch;
  p.max_query_len = mode == MXS_MODE_DECODE ? 1 : max_query_len;
  p.max_seq_len = max_seq_len;
  p.want_logits = want_logits ? 1 : 0;
  p.want_blocks = want_blocks ? 1 : 0;
  p.block = mxs::kThreads;
  const int64_t NB = ceil_div(max_seq_len, page_size);
  const int64_t capacity = (int64_t)num_cus * wg_per_cu;   // resident workgroups

  if (mode == MXS_MODE_DECODE && !want_logits) {
    // One wave per (request, 64-head group, page chunk). Chunks are sized so
    // that the waves fill the resident capacity about once (aiter #5518,
    // decode auto-CTA: host-known buckets), or the requested unit count.
    p.kernel = mxs::KID_DECODE;
    p.head_groups = (int32_t)ceil_div(num_heads, mxs::kDecodeHeads);
    const int64_t lanes = (int64_t)batch * p.head_groups;
    int64_t target_waves = parallel_unit_num > 0 ? (int64_t)parallel_unit_num * mxs::kWaves : capacity * mxs::kWaves;
    int64_t chunks = lanes > 0 ? ceil_div(target_waves, lanes) : 1;
    if (chunks > NB) chunks = NB;
    if (chunks < ceil_div(NB, mxs::kDecodeMaxPages)) chunks = ceil_div(NB, mxs::kDecodeMaxPages);
    if (chunks < 1) chunks = 1;
    p.pages_per_item = (int32_t)(NB > 0 ? ceil_div(NB, chunks) : 1);
    // a multiple of 4 chunks, so the 4 waves of a workgroup share (request,
    // head group) and can share its query tiles; surplus chunks are empty
    p.page_items = (int32_t)(ceil_div(NB > 0 ? ceil_div(NB, p.pages_per_item) : 1, mxs::kWaves) * mxs::kWaves);
    p.slot_items = 1;
    p.slots_per_item = num_heads;
    p.items = lanes * p.page_items;
    p.grid = (int32_t)ceil_div(p.items, mxs::kWaves);
  } else {
    // Work item = (request, block of query slots, chunk of pages); the grid
    // loops over the items. Logits (asked for by any call, decode included:
    // a decode request is one row with one query) come from the logits
    // kernel, prefill block scores alone from the block-score kernel.
    const bool lgk = mode == MXS_MODE_LOGITS || want_logits;
    p.kernel = lgk ? mxs::KID_LOGITS : mxs::KID_PREFILL;
    p.head_groups = 1;
    p.slots_per_item = lgk ? mxs::kLogitsSlotsPerItem : mxs::kPrefillSlotsPerItem;
    const int64_t slots = (int64_t)p.max_query_len * num_heads;
    p.slot_items = (int32_t)(slots > 0 ? ceil_div(slots, p.slots_per_item) : 0);
    const int64_t base = (int64_t)batch * p.slot_items;
    int64_t grid = parallel_unit_num > 0 ? parallel_unit_num : capacity;
    if (parallel_unit_num <= 0 && grid >= 8) grid = grid / 8 * 8;
    // pages per chunk for a chunk count: chunk starts stay 16-byte aligned
    // in the score rows, and on 128-token output windows of the logits kernel
    auto ppi_for = [&](int64_t chunks) {
      int64_t ppi = NB > 0 ? ceil_div(NB, chunks) : 1;
      if (ppi > 4) ppi = ceil_div(ppi, 4) * 4;
      if (lgk && page_size == 64) ppi = ceil_div(ppi, 2) * 2;
      return ppi;
    };
    int64_t ppi;
    if (!lgk) {
      // Block scores only: the grid strides over items ordered slot block
      // fastest. Pick the chunk count whose items spread most evenly over the
      // grid: the work is base * NB page-units, and the busiest workgroup
      // does ceil(items / grid) items of at most ppi pages each.
      ppi = ppi_for(1);
      double best = -1.0;
      for (int64_t chunks = 1; chunks <= (NB < 64 ? NB : 64); ++chunks) {
        const int64_t cp = ppi_for(chunks);
        const int64_t items = base * ceil_div(NB, cp);
        const double eff = (double)base * (double)NB / ((double)grid * (double)ceil_div(items, grid) * (double)cp);
        if (eff > best + 0.005) {
          best = eff;
          ppi = cp;
        }
      }
    } else {
      // Logits are written page chunk fastest, and each XCD's L2 should hold
      // only the part of the inputs its workgroups need. When the query slots
      // outweigh the pages they are scored against (a request's query bytes
      // above its cache bytes), the items are split across the 8 XCDs in
      // contiguous eighths (xcd_split): an XCD then reads its eighth of the
      // queries and the pages of its requests. Otherwise chunk counts go in
      // multiples of 8 (when there are pages enough): with a grid that is
      // also a multiple of 8, workgroup c only sees chunks c mod 8, so each
      // XCD reads one eighth of the pages.
      const int64_t q_bytes = (int64_t)p.max_query_len * num_heads * 128 * (q_dtype == MXS_Q_BF16 ? 2 : 1);
      const int64_t k_bytes = NB * page_size * (k_dtype == MXS_K_E4M3 ? 128 : 68);
      const int64_t want_items = parallel_unit_num > 0 ? (int64_t)parallel_unit_num * 4 : capacity * 4;
      int64_t chunks = base > 0 ? ceil_div(want_items, base) : 1;
      p.xcd_split = q_bytes > k_bytes && grid % 8 == 0 ? 1 : 0;
      if (NB >= 8 && !p.xcd_split) chunks = ceil_div(chunks, 8) * 8;
      if (chunks > NB) chunks = NB;
      if (chunks < 1) chunks = 1;
      ppi = ppi_for(chunks);
    }
    p.pages_per_item = (int32_t)ppi;
    p.page_items = (int32_t)(NB > 0 ? ceil_div(NB, ppi) : 1);
    p.items = base * p.page_items;
    if (grid > p.items) grid = p.items;
    if (grid < 1) grid = 1;
    if (p.xcd_split) {   // eight equal groups of workgroups, one per XCD
      if (grid >= 8)
        grid = grid / 8 * 8;
      else
        p.xcd_split = 0;
    }
    p.grid = (int32_t)grid;
  }
  if (p.items > INT32_MAX * (int64_t)mxs::kWaves || p.grid > INT32_MAX) return fail(MXS_EINVAL, "problem too large");
  *plan = p;
  return MXS_OK;
}

int mxs_plan_make(int32_t mode, int32_t q_dtype, int32_t k_dtype, int32_t page_size, int32_t num_heads,
                  int32_t batch, int32_t max_query_len, int32_t max_seq_len, int32_t want_logits,
                  int32_t want_blocks, int32_t parallel_unit_num, mxs_plan* plan) {
  int dev;
  DeviceInfo info;
  int rc = current_device(&dev, &info);
  if (rc != MXS_OK) return rc;
  if (q_dtype != MXS_Q_BF16 && q_dtype != MXS_Q_E4M3)
    return fail(MXS_EDTYPE, "query dtype must be bf16 or e4m3; got %d", q_dtype);
  if (check_k_dtype(k_dtype)) return MXS_EDTYPE;
  if (page_size != 64 && page_size != 128) return fail(MXS_ELAYOUT, "page_size must be 64 or 128, got %d", page_size);
  const int32_t kid = (mode == MXS_MODE_LOGITS || want_logits) ? mxs::KID_LOGITS
                      : mode == MXS_MODE_DECODE                  ? mxs::KID_DECODE
                                                                 : mxs::KID_PREFILL;
  const int occ = occupancy_cached(dev, kid, q_dtype, k_dtype, page_size, want_blocks != 0, want_logits != 0);
  return mxs_plan_make_for(mode, q_dtype, k_dtype, page_size, num_heads, batch, max_query_len, max_seq_len,
                           want_logits, want_blocks, parallel_unit_num, info.cus, occ, plan);
}

}  // extern "C"

namespace {

int check_out(const char* name, const mxs_out* o, int64_t rows, int32_t H, int64_t width) {
  if (!o || !o->ptr) return fail(MXS_EINVAL, "%s output pointer is NULL", name);
  if (!aligned(o->ptr, 4)) return fail(MXS_ELAYOUT, "%s output is not 4-byte aligned", name);
  if (o->row_stride < 0 || o->head_stride < 0) return fail(MXS_ELAYOUT, "%s output strides must be >= 0", name);
  if (H > 1 && o->head_stride < width)
    return fail(MXS_ELAYOUT, "%s output head stride %lld is narrower than its width %lld", name,
                (long long)o->head_stride, (long long)width);
  int64_t row_span;
  if (!mul_add(H - 1, o->head_stride, width, &row_span)) return fail(MXS_ELAYOUT, "%s output span overflows", name);
  if (rows > 1 && o->row_stride < row_span)
    return fail(MXS_ELAYOUT, "%s output row stride %lld is narrower than one row (%lld)", name,
                (long long)o->row_stride, (long long)row_span);
  int64_t span;
  if (!mul_add(rows - 1, o->row_stride, row_span, &span) || span > INT64_MAX / 4)
    return fail(MXS_ELAYOUT, "%s output span overflows", name);
  return MXS_OK;
}

// The structural invariants the kernels rely on (a caller may pass a plan
// it has modified or made for another device).
bool plan_consistent(const mxs_plan& p, int mode, int32_t H, int32_t B, int32_t max_query_len, int64_t NB) {
  if (p.block != mxs::kThreads || p.grid < 1 || p.pages_per_item < 1 || p.page_items < 1) return false;
  if ((int64_t)p.page_items * p.pages_per_item < NB) return false;
  if (mode == MXS_MODE_DECODE && !p.want_logits) {
    return p.kernel == mxs::KID_DECODE && p.xcd_split == 0 && p.head_groups == ceil_div(H, mxs::kDecodeHeads) &&
           p.pages_per_item <= mxs::kDecodeMaxPages && p.page_items % mxs::kWaves == 0 &&
           p.items == (int64_t)B * p.head_groups * p.page_items && (int64_t)p.grid * mxs::kWaves == p.items;
  }
  const bool lgk = mode == MXS_MODE_LOGITS || p.want_logits;
  const int32_t kid = lgk ? mxs::KID_LOGITS : mxs::KID_PREFILL;
  const int64_t slots = (int64_t)max_query_len * H;
  if (p.xcd_split != 0 && (p.xcd_split != 1 || !lgk || p.grid % 8 != 0)) return false;
  return p.kernel == kid && p.slots_per_item == (lgk ? mxs::kLogitsSlotsPerItem : mxs::kPrefillSlotsPerItem) &&
         p.slot_items == (slots > 0 ? ceil_div(slots, p.slots_per_item) : 0) &&
         p.items == (int64_t)B * p.slot_items * p.page_items && p.grid <= (p.items > 0 ? p.items : 1);
}

int score(int mode, const mxs_query* q, const mxs_kcache* k, const mxs_batch* bt, float sm_scale,
          const mxs_out* bs, const mxs_out* lg, const mxs_plan* plan_in, void* stream) {
  if (!q || !k || !bt) return fail(MXS_EINVAL, "query, cache and batch descriptors must not be NULL");
  if (q->dtype != MXS_Q_BF16 && q->dtype != MXS_Q_E4M3)
    return fail(MXS_EDTYPE, "query dtype must be bf16 (%d) or e4m3 (%d); got %d (fp16 is refused)", MXS_Q_BF16,
                MXS_Q_E4M3, q->dtype);
  if (q->num_heads < 1) return fail(MXS_EINVAL, "num_heads must be >= 1, got %d", q->num_heads);
  if (k->page_size != 64 && k->page_size != 128)
    return fail(MXS_ELAYOUT, "page_size must be 64 or 128, got %d", k->page_size);
  if (check_k_dtype(k->k_dtype)) return MXS_EDTYPE;
  if (!(std::isfinite(sm_scale) && sm_scale > 0.0f)) return fail(MXS_EINVAL, "sm_scale must be finite and > 0");
  if (bt->batch < 0 || bt->max_seq_len < 0) return fail(MXS_EINVAL, "batch and max_seq_len must be >= 0");
  if (bt->max_seq_len > mxs::kMaxSeqLen)
    return fail(MXS_EINVAL, "max_seq_len %d is above the limit %d", bt->max_seq_len, mxs::kMaxSeqLen);
  const bool decode = mode == MXS_MODE_DECODE;
  if (!decode && (bt->total_rows < 0 || bt->max_query_len < 0))
    return fail(MXS_EINVAL, "total_rows and max_query_len must be >= 0");
  const bool want_bs = bs && bs->ptr;
  const bool want_lg = lg && lg->ptr;

  const int32_t H = q->num_heads, P = k->page_size;
  const int64_t rows = decode ? bt->batch : bt->total_rows;
  const int64_t NB = ceil_div(bt->max_seq_len, P);
  // Nothing to write: no rows or an empty window. The outputs then hold no
  // element and may be NULL (an empty tensor's data pointer).
  if (rows == 0 || bt->max_seq_len == 0 || bt->batch == 0) return MXS_OK;
  if (mode != MXS_MODE_LOGITS && !want_bs) return fail(MXS_EINVAL, "block_scores output is required");
  if (mode == MXS_MODE_LOGITS && !want_lg) return fail(MXS_EINVAL, "logits output is required in logits mode");
  // query
  const int64_t es = q->dtype == MXS_Q_BF16 ? 2 : 1;
  if (!q->ptr) return fail(MXS_EINVAL, "query pointer is NULL");
  if (!aligned(q->ptr, 16)) return fail(MXS_ELAYOUT, "query rows must be 16-byte aligned");
  if (q->row_stride < 0 || q->head_stride < 0) return fail(MXS_ELAYOUT, "query strides must be >= 0");
  if ((q->row_stride * es) % 16 || (q->head_stride * es) % 16)
    return fail(MXS_ELAYOUT, "query row and head strides must be multiples of 16 bytes (misaligned query rows)");
  // cache
  {
    const int rck = check_kcache_views(k);
    if (rck != MXS_OK) return rck;
  }
  // batch metadata
  if (!bt->block_table || !bt->seq_lens) return fail(MXS_EINVAL, "block_table and seq_lens must not be NULL");
  if (!decode && (!bt->cu_seqlens_q || !bt->prefix_lens))
    return fail(MXS_EINVAL, "cu_seqlens_q and prefix_lens must not be NULL");
  if (!aligned(bt->block_table, 4) || !aligned(bt->seq_lens, 4) ||
      (!decode && (!aligned(bt->cu_seqlens_q, 4) || !aligned(bt->prefix_lens, 4))))
    return fail(MXS_ELAYOUT, "int32 metadata must be 4-byte aligned");
  if (bt->bt_width < NB)
    return fail(MXS_ELAYOUT, "block table width %d is narrower than ceil(max_seq_len / page_size) = %lld",
                bt->bt_width, (long long)NB);
  if (bt->batch > 1 && bt->bt_row_stride < bt->bt_width)
    return fail(MXS_ELAYOUT, "block table row stride %lld is smaller than its width %d", (long long)bt->bt_row_stride,
                bt->bt_width);
  // outputs
  if (want_bs) {
    int rc = check_out("block_scores", bs, rows, H, NB);
    if (rc) return rc;
  }
  if (want_lg) {
    int rc = check_out("logits", lg, rows, H, bt->max_seq_len);
    if (rc) return rc;
  }
  // device and plan
  int dev;
  DeviceInfo info;
  int rc = current_device(&dev, &info);
  if (rc != MXS_OK) return rc;
  mxs_plan plan;
  if (plan_in) {
    if (plan_in->mode != mode || plan_in->q_dtype != q->dtype || plan_in->k_dtype != k->k_dtype ||
        plan_in->page_size != P || plan_in->num_heads != H ||
        plan_in->batch != bt->batch || plan_in->max_seq_len != bt->max_seq_len ||
        (!decode && plan_in->max_query_len != bt->max_query_len) || plan_in->want_logits != (want_lg ? 1 : 0) ||
        plan_in->want_blocks != (want_bs ? 1 : 0))
      return fail(MXS_EINVAL, "the plan was made for different shapes or outputs");
    plan = *plan_in;
  } else {
    rc = mxs_plan_make(mode, q->dtype, k->k_dtype, P, H, bt->batch, decode ? 1 : bt->max_query_len, bt->max_seq_len,
                       want_lg, want_bs, 0, &plan);
    if (rc != MXS_OK) return rc;
  }
  if (!plan_consistent(plan, mode, H, bt->batch, decode ? 1 : bt->max_query_len, NB))
    return fail(MXS_EINVAL, "the plan's work decomposition is inconsistent with its shapes");
  if (plan.items == 0) return MXS_OK;

  mxs::KArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = static_cast<const uint8_t*>(q->ptr);
  a.q_row_stride = q->row_stride * es;
  a.q_head_stride = q->head_stride * es;
  a.H = H;
  a.kd = static_cast<const uint8_t*>(k->data);
  a.kd_page_stride = k->data_page_stride;
  a.ks = k->k_dtype == MXS_K_E4M3 ? nullptr : static_cast<const uint8_t*>(k->scale);
  a.ks_page_stride = k->scale_page_stride;
  a.bt = bt->block_table;
  a.bt_stride = bt->bt_row_stride;
  a.cu = bt->cu_seqlens_q;
  a.seq = bt->seq_lens;
  a.prefix = bt->prefix_lens;
  a.B = bt->batch;
  a.max_seq_len = bt->max_seq_len;
  a.NB = (int32_t)NB;
  a.sm_scale = sm_scale;
  if (want_bs) {
    a.bs = bs->ptr;
    a.bs_row_stride = bs->row_stride;
    a.bs_head_stride = bs->head_stride;
    // widest store every block-score row allows: 16, 8 or 4 bytes
    a.vec_bs = aligned(bs->ptr, 16) && bs->row_stride % 4 == 0 && bs->head_stride % 4 == 0  ? 4
               : aligned(bs->ptr, 8) && bs->row_stride % 2 == 0 && bs->head_stride % 2 == 0 ? 2
                                                                                             : 1;
  }
  if (want_lg) {
    a.lg = lg->ptr;
    a.lg_row_stride = lg->row_stride;
    a.lg_head_stride = lg->head_stride;
    a.vec_lg = aligned(lg->ptr, 16) && lg->row_stride % 4 == 0 && lg->head_stride % 4 == 0;
  }
  a.slots_per_item = plan.slots_per_item;
  a.pages_per_item = plan.pages_per_item;
  a.slot_items = plan.slot_items;
  a.page_items = plan.page_items;
  a.head_groups = plan.head_groups;
  a.items = plan.items;
  a.decode_rows = decode && plan.kernel == mxs::KID_LOGITS ? 1 : 0;
  a.xcd_split = plan.xcd_split;
  hipError_t e = mxs::launch(plan, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MXS_EDEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  return MXS_OK;
}

}  // namespace

extern "C" {

int mxs_score_prefill(const mxs_query* q, const mxs_kcache* k, const mxs_batch* batch, float sm_scale,
                      const mxs_out* block_scores, const mxs_out* logits, const mxs_plan* plan, void* stream) {
  return score(MXS_MODE_PREFILL, q, k, batch, sm_scale, block_scores, logits, plan, stream);
}

int mxs_score_decode(const mxs_query* q, const mxs_kcache* k, const mxs_batch* batch, float sm_scale,
                     const mxs_out* block_scores, const mxs_out* logits, const mxs_plan* plan, void* stream) {
  return score(MXS_MODE_DECODE, q, k, batch, sm_scale, block_scores, logits, plan, stream);
}

int mxs_score_logits(const mxs_query* q, const mxs_kcache* k, const mxs_batch* batch, float sm_scale,
                     const mxs_out* logits, const mxs_out* block_scores, const mxs_plan* plan, void* stream) {
  return score(MXS_MODE_LOGITS, q, k, batch, sm_scale, block_scores, logits, plan, stream);
}

}  // extern "C"
