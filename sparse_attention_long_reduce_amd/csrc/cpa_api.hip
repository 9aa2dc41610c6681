// C ABI: host-side argument checks, work decomposition and launches (see include/cpa.h).
#include "cpa.h"
#include "cpa_internal.h"

#include <climits>
#include <cmath>
#include <mutex>

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" size_t cpa_split_workspace_bytes(int total_q, int Hq, int d, int table_cap, int split_pages);

namespace {
// V pool description: strides in elements; v_row_stride is the token stride of token-major
// pages (dim contiguous) or the dim stride of dim-major pages (tokens contiguous)
struct VLayout {
  int64_t page_stride, head_stride, row_stride;
  bool dmajor;
};

// Largest stride (elements) and head count the entry points take: far beyond any pool that fits
// in memory, and small enough that no size product the checks or the kernels form overflows.
constexpr int64_t kMaxStride = (int64_t)1 << 40;
constexpr int kMaxHeads = 65536;

// Workgroups of a prefill launch with n_splits ranges per tile, as the kernels' grid computes
// it, in 64 bits (the launch takes at most INT_MAX).
int64_t prefill_workgroups(const cpa::PrefillArgs& a, int64_t n_splits) {
  const int64_t groups = a.n_groups;
  const int64_t slots = a.xcd_remap ? 8 * ((groups + 7) / 8) : groups;
  return slots * a.tiles_per_group * n_splits;
}

// Checks the arguments of a prefill call and fills the launch arguments (no HIP call).
// *nothing: the call has no work (B == 0 or max_chunk_len == 0).
cpa_status prepare_prefill(const void* q, cpa_dtype dtype, const void* k_pages,
                           const void* v_pages, int64_t page_stride, int64_t head_stride,
                           int64_t token_stride, const VLayout& vl, int64_t n_pages, const int32_t* page_map,
                           int page_map_stride, const int32_t* tables, int table_cap,
                           const int32_t* counts, const int32_t* cu_q,
                           const int32_t* prefix_len, int B, int Hq, int Hkv, int d,
                           int max_chunk_len, float sm_scale, void* o, float* lse,
                           cpa::PrefillArgs& a, bool* nothing, int kv_elem_bytes = 0,
                           bool with_tables = true) {
  *nothing = false;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || max_chunk_len < 0 || table_cap < 0 || n_pages < 0)
    return CPA_ERR_SHAPE;
  if (Hq % Hkv != 0 || Hq > kMaxHeads) return CPA_ERR_SHAPE;
  if (!(sm_scale >= 0.f) || std::isinf(sm_scale)) return CPA_ERR_SHAPE;
  if (dtype != CPA_F32 && dtype != CPA_BF16) return CPA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return CPA_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (B == 0 || max_chunk_len == 0) {
    *nothing = true;
    return CPA_OK;
  }
  if (page_map_stride < 1) return CPA_ERR_SHAPE;
  // the kernels stage page 0 of the pool for copy slots that have no page to fill, so a call
  // with work needs a pool of at least one page
  if (n_pages < 1) return CPA_ERR_SHAPE;
  if (token_stride > kMaxStride || head_stride > kMaxStride || page_stride > kMaxStride ||
      vl.row_stride > kMaxStride || vl.head_stride > kMaxStride || vl.page_stride > kMaxStride)
    return CPA_ERR_SHAPE;
  if (token_stride < d || head_stride < 64 * token_stride || page_stride < (int64_t)Hkv * head_stride)
    return CPA_ERR_SHAPE;
  const int64_t v_rows = vl.dmajor ? d : 64, v_row_len = vl.dmajor ? 64 : d;
  if (vl.row_stride < v_row_len || vl.head_stride < v_rows * vl.row_stride ||
      vl.page_stride < (int64_t)Hkv * vl.head_stride)
    return CPA_ERR_SHAPE;
  if (!q || !k_pages || !v_pages || !page_map || !cu_q || !prefix_len || !o) return CPA_ERR_NULL;
  if (with_tables && (!counts || (table_cap > 0 && !tables))) return CPA_ERR_NULL;
  // bytes per pool element: that of q's dtype unless the pools hold another format (fp8)
  const int eb = kv_elem_bytes > 0 ? kv_elem_bytes : dtype == CPA_BF16 ? 2 : 4;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o)) return CPA_ERR_ALIGN;
  if ((token_stride * eb) % 16 || (head_stride * eb) % 16 || (page_stride * eb) % 16) return CPA_ERR_ALIGN;
  if ((vl.row_stride * eb) % 16 || (vl.head_stride * eb) % 16 || (vl.page_stride * eb) % 16) return CPA_ERR_ALIGN;

  a = cpa::PrefillArgs{};
  a.q = q; a.k = k_pages; a.v = v_pages;
  a.page_stride = page_stride; a.head_stride = head_stride; a.token_stride = token_stride;
  a.v_page_stride = vl.page_stride; a.v_head_stride = vl.head_stride; a.v_row_stride = vl.row_stride;
  a.v_dmajor = vl.dmajor ? 1 : 0;
  a.n_pages = n_pages;
  a.page_map = page_map; a.page_map_stride = page_map_stride;
  a.tables = tables; a.table_cap = table_cap; a.counts = counts;
  a.cu_q = cu_q; a.prefix_len = prefix_len;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.max_chunk_len = max_chunk_len;
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / std::sqrt((float)d);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_scale = 1.0f;
  a.o = o; a.lse = lse;
  a.G = G;
  const int64_t nqb_max = (max_chunk_len + CPA_BLOCK - 1) / CPA_BLOCK;
  const int64_t tiles = (nqb_max * G + cpa::PAIRS_PER_TILE - 1) / cpa::PAIRS_PER_TILE;
  if (tiles > INT_MAX || (int64_t)B * Hkv > INT_MAX) return CPA_ERR_SHAPE;
  a.tiles_per_group = (int)tiles;
  a.n_groups = B * Hkv;
  a.xcd_remap = a.n_groups >= 8 ? 1 : 0;
  a.n_splits = 1;
  if (prefill_workgroups(a, 1) > INT_MAX) return CPA_ERR_SHAPE;
  return CPA_OK;
}

// Runs a prepared prefill split into ceil(table_cap / split_pages) ranges per tile plus the
// merge (the plain path when that is one range); defined with the split entry points below.
cpa_status launch_split(cpa::PrefillArgs& a, cpa_dtype dtype, int64_t token_stride, const VLayout& vl,
                        int table_cap, int Hq, int d, void* o, float* lse, int total_q, int split_pages,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

}  // namespace

extern "C" {

const char* cpa_status_string(cpa_status s) {
  switch (s) {
    case CPA_OK: return "ok";
    case CPA_ERR_NULL: return "a required pointer is NULL";
    case CPA_ERR_SHAPE: return "invalid or inconsistent size";
    case CPA_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case CPA_ERR_UNSUPPORTED: return "unsupported dtype, head dim or path";
    case CPA_ERR_CAPACITY: return "table capacity smaller than the KV-block count, or workspace too small";
    case CPA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int cpa_version(void) { return 10000; }

cpa_status cpa_build_block_tables(const uint8_t* masks, int B, int Hq, int Hkv, int nqb_max,
                                  int nkvb_max, const int32_t* prefix_blocks,
                                  const int32_t* chunk_blocks, int32_t* tables, int table_cap,
                                  int32_t* counts, hipStream_t stream) {
  if (B < 0 || Hq < 0 || Hkv <= 0 || nqb_max < 0 || nkvb_max < 0 || table_cap < 0) return CPA_ERR_SHAPE;
  if (Hq % Hkv != 0 || Hq > kMaxHeads || (int64_t)B * Hkv > INT_MAX) return CPA_ERR_SHAPE;
  if (nkvb_max > CPA_MAX_KV_BLOCKS) return CPA_ERR_SHAPE;
  if (table_cap < nkvb_max) return CPA_ERR_CAPACITY;
  if (B == 0) return CPA_OK;
  if (!prefix_blocks || !chunk_blocks || !counts) return CPA_ERR_NULL;
  if (table_cap > 0 && !tables) return CPA_ERR_NULL;
  if (Hq > 0 && nqb_max > 0 && nkvb_max > 0 && !masks) return CPA_ERR_NULL;
  cpa::UnionArgs a{masks, B, Hq, Hkv, nqb_max, nkvb_max, prefix_blocks, chunk_blocks, tables, table_cap, counts,
                   nullptr, 0, 0};
  return cpa::launch_block_union(a, stream) == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}

cpa_status cpa_build_block_tables_bits(const uint64_t* mask_bits, int B, int Hq, int Hkv, int nqb_max,
                                       int nkvb_max, int mask_words, const int32_t* prefix_blocks,
                                       const int32_t* chunk_blocks, int32_t* tables, int table_cap,
                                       int32_t* counts, hipStream_t stream) {
  if (B < 0 || Hq < 0 || Hkv <= 0 || nqb_max < 0 || nkvb_max < 0 || table_cap < 0 || mask_words < 0)
    return CPA_ERR_SHAPE;
  if (Hq % Hkv != 0 || Hq > kMaxHeads || (int64_t)B * Hkv > INT_MAX) return CPA_ERR_SHAPE;
  if (nkvb_max > CPA_MAX_KV_BLOCKS) return CPA_ERR_SHAPE;
  if (mask_words < (nkvb_max + 63) / 64) return CPA_ERR_SHAPE;
  if (table_cap < nkvb_max) return CPA_ERR_CAPACITY;
  if (B == 0) return CPA_OK;
  if (!prefix_blocks || !chunk_blocks || !counts) return CPA_ERR_NULL;
  if (table_cap > 0 && !tables) return CPA_ERR_NULL;
  if (Hq > 0 && nqb_max > 0 && nkvb_max > 0 && !mask_bits) return CPA_ERR_NULL;
  if (((uintptr_t)mask_bits & 7u) != 0) return CPA_ERR_ALIGN;
  cpa::UnionArgs a{nullptr, B, Hq, Hkv, nqb_max, nkvb_max, prefix_blocks, chunk_blocks, tables, table_cap, counts,
                   reinterpret_cast<const unsigned long long*>(mask_bits), mask_words, 1};
  return cpa::launch_block_union(a, stream) == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}

cpa_status cpa_chunked_prefill(const void* q, cpa_dtype dtype, const void* k_pages,
                               const void* v_pages, int64_t page_stride, int64_t head_stride,
                               int64_t token_stride, int64_t n_pages, const int32_t* page_map,
                               int page_map_stride, const int32_t* tables, int table_cap,
                               const int32_t* counts, const int32_t* cu_q,
                               const int32_t* prefix_len, int B, int Hq, int Hkv, int d,
                               int max_chunk_len, float sm_scale, void* o, float* lse,
                               hipStream_t stream) {
  cpa::PrefillArgs a;
  bool nothing;
  const VLayout vl{page_stride, head_stride, token_stride, false};
  const cpa_status st = prepare_prefill(q, dtype, k_pages, v_pages, page_stride, head_stride, token_stride, vl,
                                        n_pages, page_map, page_map_stride, tables, table_cap, counts, cu_q,
                                        prefix_len, B, Hq, Hkv, d, max_chunk_len, sm_scale, o, lse, a, &nothing);
  if (st != CPA_OK || nothing) return st;
  return cpa::launch_prefill(a, dtype == CPA_BF16, d, stream) == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}

cpa_status cpa_append_kv(const void* k_new, const void* v_new, cpa_dtype dtype, void* k_pages,
                         int64_t page_stride, int64_t head_stride, int64_t token_stride, void* v_pages,
                         int v_dim_major, int64_t v_page_stride, int64_t v_head_stride, int64_t v_row_stride,
                         int64_t n_pages, const int32_t* page_map, int page_map_stride, const int32_t* cu_q,
                         const int32_t* prefix_len, int B, int Hkv, int d, int max_chunk_len,
                         hipStream_t stream) {
  if (B < 0 || Hkv <= 0 || Hkv > kMaxHeads || max_chunk_len < 0 || n_pages < 0) return CPA_ERR_SHAPE;
  if (dtype != CPA_F32 && dtype != CPA_BF16 && dtype != CPA_FP8_E4M3) return CPA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return CPA_ERR_UNSUPPORTED;
  if (v_dim_major != 0 && v_dim_major != 1) return CPA_ERR_SHAPE;
  if (B == 0 || max_chunk_len == 0) return CPA_OK;
  if (page_map_stride < 1) return CPA_ERR_SHAPE;
  if (token_stride > kMaxStride || head_stride > kMaxStride || page_stride > kMaxStride ||
      v_row_stride > kMaxStride || v_head_stride > kMaxStride || v_page_stride > kMaxStride)
    return CPA_ERR_SHAPE;
  if ((int64_t)B * ((max_chunk_len + 63) / 64) * Hkv > INT_MAX) return CPA_ERR_SHAPE;   // workgroups
  if (token_stride < d || head_stride < 64 * token_stride || page_stride < (int64_t)Hkv * head_stride)
    return CPA_ERR_SHAPE;
  const int64_t v_rows = v_dim_major ? d : 64, v_row_len = v_dim_major ? 64 : d;
  if (v_row_stride < v_row_len || v_head_stride < v_rows * v_row_stride ||
      v_page_stride < (int64_t)Hkv * v_head_stride)
    return CPA_ERR_SHAPE;
  if (!k_new || !v_new || !k_pages || !v_pages || !page_map || !cu_q || !prefix_len) return CPA_ERR_NULL;
  const int eb = dtype == CPA_BF16 ? 2 : dtype == CPA_FP8_E4M3 ? 1 : 4;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pages) || !aligned16(v_pages)) return CPA_ERR_ALIGN;
  if ((token_stride * eb) % 16 || (head_stride * eb) % 16 || (page_stride * eb) % 16) return CPA_ERR_ALIGN;
  if ((v_row_stride * eb) % 16 || (v_head_stride * eb) % 16 || (v_page_stride * eb) % 16) return CPA_ERR_ALIGN;
  if ((long long)B * ((max_chunk_len + 63) / 64) * Hkv > 0x7fffffffLL) return CPA_ERR_SHAPE;
  cpa::AppendArgs a{};
  a.k_new = k_new; a.v_new = v_new; a.k_pages = k_pages; a.v_pages = v_pages;
  a.page_stride = page_stride; a.head_stride = head_stride; a.token_stride = token_stride; a.n_pages = n_pages;
  a.v_page_stride = v_page_stride; a.v_head_stride = v_head_stride; a.v_row_stride = v_row_stride;
  a.v_dmajor = v_dim_major;
  a.page_map = page_map; a.page_map_stride = page_map_stride;
  a.cu_q = cu_q; a.prefix_len = prefix_len;
  a.B = B; a.Hkv = Hkv; a.max_chunk_len = max_chunk_len;
  return cpa::launch_kv_append(a, eb, d, stream) == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}

cpa_status cpa_chunked_prefill_fp8kv(const void* q, const void* k_pages, const void* v_pages, int64_t page_stride,
                                     int64_t head_stride, int64_t token_stride, int v_dim_major,
                                     int64_t v_page_stride, int64_t v_head_stride, int64_t v_row_stride,
                                     float k_scale, float v_scale, int64_t n_pages, const int32_t* page_map,
                                     int page_map_stride, const int32_t* tables, int table_cap,
                                     const int32_t* counts, const int32_t* cu_q, const int32_t* prefix_len, int B,
                                     int Hq, int Hkv, int d, int max_chunk_len, float sm_scale, void* o, float* lse,
                                     int total_q, int split_pages, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || std::isinf(k_scale) || std::isinf(v_scale)) return CPA_ERR_SHAPE;
  if (v_dim_major != 0 && v_dim_major != 1) return CPA_ERR_SHAPE;
  if (split_pages >= 1 && total_q < 0) return CPA_ERR_SHAPE;
  cpa::PrefillArgs a;
  bool nothing;
  const VLayout vl{v_page_stride, v_head_stride, v_row_stride, v_dim_major == 1};
  const cpa_status st = prepare_prefill(q, CPA_BF16, k_pages, v_pages, page_stride, head_stride, token_stride, vl,
                                        n_pages, page_map, page_map_stride, tables, table_cap, counts, cu_q,
                                        prefix_len, B, Hq, Hkv, d, max_chunk_len, sm_scale, o, lse, a, &nothing,
                                        /*kv_elem_bytes=*/1);
  if (st != CPA_OK || nothing) return st;
  a.kv_fp8 = 1;
  a.scale_log2 *= k_scale;   // scores of the stored values times the K scale
  a.out_scale = v_scale;     // the output is linear in V (each split range's partial is scaled too)
  if (split_pages >= 1)
    return launch_split(a, CPA_BF16, token_stride, vl, table_cap, Hq, d, o, lse, total_q, split_pages, workspace,
                        workspace_bytes, stream);
  // either V layout: the direct-to-LDS kernel stages codes and converts each page once per
  // workgroup; pools whose strides overflow its 32-bit offsets go to the register-staged kernel
  return cpa::launch_prefill(a, true, d, stream) == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}

cpa_status cpa_build_block_plans(const uint8_t* masks, int B, int Hq, int nqb_max, int nkvb_max,
                                 const int32_t* prefix_blocks, const int32_t* chunk_blocks, int32_t* plans,
                                 int plan_cap, int32_t* plan_counts, hipStream_t stream) {
  if (B < 0 || Hq < 0 || nqb_max < 0 || nkvb_max < 0 || plan_cap < 0) return CPA_ERR_SHAPE;
  if (nkvb_max > CPA_MAX_KV_BLOCKS) return CPA_ERR_SHAPE;
  if (plan_cap < nkvb_max) return CPA_ERR_CAPACITY;
  if ((long long)B * Hq * nqb_max == 0) return CPA_OK;
  if (!prefix_blocks || !chunk_blocks || !plan_counts) return CPA_ERR_NULL;
  if (plan_cap > 0 && !plans) return CPA_ERR_NULL;
  if (nkvb_max > 0 && !masks) return CPA_ERR_NULL;
  cpa::PlanArgs a{masks, B, Hq, nqb_max, nkvb_max, prefix_blocks, chunk_blocks, plans, plan_cap, plan_counts};
  return cpa::launch_block_plans(a, stream) == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}

cpa_status cpa_chunked_prefill_direct(const void* q, cpa_dtype dtype, const void* k_pages, int64_t page_stride,
                                      int64_t head_stride, int64_t token_stride, const void* v_pages,
                                      int64_t v_page_stride, int64_t v_head_stride, int64_t v_dim_stride,
                                      int64_t n_pages, const int32_t* page_map, int page_map_stride,
                                      const int32_t* plans, int plan_cap, const int32_t* plan_counts,
                                      int nqb_max, const int32_t* cu_q, const int32_t* prefix_len, int B, int Hq,
                                      int Hkv, int d, int max_chunk_len, float sm_scale, void* o, float* lse,
                                      hipStream_t stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || max_chunk_len < 0 || plan_cap < 0 || n_pages < 0 || nqb_max < 0)
    return CPA_ERR_SHAPE;
  if (Hq % Hkv != 0 || Hq > kMaxHeads || (int64_t)B * Hkv > INT_MAX) return CPA_ERR_SHAPE;
  if (!(sm_scale >= 0.f) || std::isinf(sm_scale)) return CPA_ERR_SHAPE;
  if (dtype != CPA_BF16) return CPA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return CPA_ERR_UNSUPPORTED;
  if (nqb_max < (max_chunk_len + CPA_BLOCK - 1) / CPA_BLOCK) return CPA_ERR_SHAPE;
  if (B == 0 || max_chunk_len == 0) return CPA_OK;
  if (page_map_stride < 1) return CPA_ERR_SHAPE;
  if (token_stride > kMaxStride || head_stride > kMaxStride || page_stride > kMaxStride ||
      v_dim_stride > kMaxStride || v_head_stride > kMaxStride || v_page_stride > kMaxStride)
    return CPA_ERR_SHAPE;
  if (token_stride < d || head_stride < 64 * token_stride || page_stride < (int64_t)Hkv * head_stride)
    return CPA_ERR_SHAPE;
  if (v_dim_stride < 64 || v_head_stride < (int64_t)d * v_dim_stride || v_page_stride < (int64_t)Hkv * v_head_stride)
    return CPA_ERR_SHAPE;
  if (!q || !k_pages || !v_pages || !page_map || !plan_counts || !cu_q || !prefix_len || !o) return CPA_ERR_NULL;
  if (plan_cap > 0 && !plans) return CPA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o)) return CPA_ERR_ALIGN;
  if ((token_stride * 2) % 16 || (head_stride * 2) % 16 || (page_stride * 2) % 16) return CPA_ERR_ALIGN;
  if ((v_dim_stride * 2) % 16 || (v_head_stride * 2) % 16 || (v_page_stride * 2) % 16) return CPA_ERR_ALIGN;
  cpa::DirectArgs a{};
  a.q = q; a.k = k_pages; a.v = v_pages;
  a.page_stride = page_stride; a.head_stride = head_stride; a.token_stride = token_stride;
  a.v_page_stride = v_page_stride; a.v_head_stride = v_head_stride; a.v_dim_stride = v_dim_stride;
  a.n_pages = n_pages; a.page_map = page_map; a.page_map_stride = page_map_stride;
  a.plans = plans; a.plan_cap = plan_cap; a.plan_counts = plan_counts;
  a.cu_q = cu_q; a.prefix_len = prefix_len;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.max_chunk_len = max_chunk_len; a.nqb_max = nqb_max;
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / std::sqrt((float)d);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o = o; a.lse = lse;
  a.xcd_remap = B * Hkv >= 8 ? 1 : 0;
  return cpa::launch_prefill_direct(a, d, stream) == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}

size_t cpa_split_workspace_bytes(int total_q, int Hq, int d, int table_cap, int split_pages) {
  if (total_q <= 0 || Hq <= 0 || d <= 0 || table_cap <= 0 || split_pages <= 0) return 0;
  const size_t n_splits = ((size_t)table_cap + split_pages - 1) / split_pages;
  if (n_splits <= 1) return 0;
  return n_splits * (size_t)total_q * (size_t)Hq * (size_t)(d + 1) * sizeof(float);
}

}  // extern "C"

namespace {
// The split-KV launches for prepared arguments a: ranges of split_pages pages of tables that
// hold at most table_cap ids, the partials in the workspace, then the merge.
cpa_status launch_split(cpa::PrefillArgs& a, cpa_dtype dtype, int64_t token_stride, const VLayout& vl,
                        int table_cap, int Hq, int d, void* o, float* lse, int total_q, int split_pages,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int64_t n_splits = ((int64_t)table_cap + split_pages - 1) / split_pages;
  if (n_splits <= 1)   // one range: the plain path
    return cpa::launch_prefill(a, dtype == CPA_BF16, d, stream) == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
  if (dtype != CPA_BF16 || token_stride > (1 << 24) || vl.row_stride > (1 << 24)) return CPA_ERR_UNSUPPORTED;
  if (total_q == 0) return CPA_OK;
  const size_t need = cpa_split_workspace_bytes(total_q, Hq, d, table_cap, split_pages);
  if (workspace == nullptr) return CPA_ERR_NULL;
  if (!aligned16(workspace)) return CPA_ERR_ALIGN;
  if (workspace_bytes < need) return CPA_ERR_CAPACITY;
  if (prefill_workgroups(a, n_splits) > INT_MAX) return CPA_ERR_SHAPE;
  a.n_splits = (int)n_splits;
  a.split_pages = split_pages;
  a.total_q = total_q;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = a.part_o + (size_t)n_splits * total_q * Hq * d;
  if (cpa::launch_prefill(a, true, d, stream) != hipSuccess) return CPA_ERR_LAUNCH;
  cpa::MergeArgs m{a.part_o, a.part_lse, a.n_splits, total_q, Hq, o, lse};
  return cpa::launch_split_merge(m, d, stream) == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}

// the split-KV call for either V layout (split_pages >= 1)
cpa_status prefill_split(const void* q, cpa_dtype dtype, const void* k_pages, const void* v_pages,
                         int64_t page_stride, int64_t head_stride, int64_t token_stride, const VLayout& vl,
                         int64_t n_pages, const int32_t* page_map, int page_map_stride,
                         const int32_t* tables, int table_cap, const int32_t* counts, const int32_t* cu_q,
                         const int32_t* prefix_len, int B, int Hq, int Hkv, int d, int max_chunk_len,
                         float sm_scale, void* o, float* lse, int total_q, int split_pages, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (split_pages <= 0 || total_q < 0) return CPA_ERR_SHAPE;
  cpa::PrefillArgs a;
  bool nothing;
  const cpa_status st = prepare_prefill(q, dtype, k_pages, v_pages, page_stride, head_stride, token_stride, vl,
                                        n_pages, page_map, page_map_stride, tables, table_cap, counts, cu_q,
                                        prefix_len, B, Hq, Hkv, d, max_chunk_len, sm_scale, o, lse, a, &nothing);
  if (st != CPA_OK || nothing) return st;
  return launch_split(a, dtype, token_stride, vl, table_cap, Hq, d, o, lse, total_q, split_pages, workspace,
                      workspace_bytes, stream);
}
}  // namespace

extern "C" {

cpa_status cpa_chunked_prefill_split(const void* q, cpa_dtype dtype, const void* k_pages,
                                     const void* v_pages, int64_t page_stride, int64_t head_stride,
                                     int64_t token_stride, int64_t n_pages, const int32_t* page_map,
                                     int page_map_stride, const int32_t* tables, int table_cap,
                                     const int32_t* counts, const int32_t* cu_q,
                                     const int32_t* prefix_len, int B, int Hq, int Hkv, int d,
                                     int max_chunk_len, float sm_scale, void* o, float* lse,
                                     int total_q, int split_pages, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  const VLayout vl{page_stride, head_stride, token_stride, false};
  return prefill_split(q, dtype, k_pages, v_pages, page_stride, head_stride, token_stride, vl, n_pages, page_map,
                       page_map_stride, tables, table_cap, counts, cu_q, prefix_len, B, Hq, Hkv, d, max_chunk_len,
                       sm_scale, o, lse, total_q, split_pages, workspace, workspace_bytes, stream);
}

cpa_status cpa_chunked_prefill_vt(const void* q, cpa_dtype dtype, const void* k_pages, int64_t page_stride,
                                  int64_t head_stride, int64_t token_stride, const void* v_pages,
                                  int64_t v_page_stride, int64_t v_head_stride, int64_t v_dim_stride,
                                  int64_t n_pages, const int32_t* page_map, int page_map_stride,
                                  const int32_t* tables, int table_cap, const int32_t* counts,
                                  const int32_t* cu_q, const int32_t* prefix_len, int B, int Hq, int Hkv,
                                  int d, int max_chunk_len, float sm_scale, void* o, float* lse, int total_q,
                                  int split_pages, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  const VLayout vl{v_page_stride, v_head_stride, v_dim_stride, true};
  if (split_pages > 0)
    return prefill_split(q, dtype, k_pages, v_pages, page_stride, head_stride, token_stride, vl, n_pages,
                         page_map, page_map_stride, tables, table_cap, counts, cu_q, prefix_len, B, Hq, Hkv, d,
                         max_chunk_len, sm_scale, o, lse, total_q, split_pages, workspace, workspace_bytes,
                         stream);
  if (total_q < 0) return CPA_ERR_SHAPE;
  cpa::PrefillArgs a;
  bool nothing;
  const cpa_status st = prepare_prefill(q, dtype, k_pages, v_pages, page_stride, head_stride, token_stride, vl,
                                        n_pages, page_map, page_map_stride, tables, table_cap, counts, cu_q,
                                        prefix_len, B, Hq, Hkv, d, max_chunk_len, sm_scale, o, lse, a, &nothing);
  if (st != CPA_OK || nothing) return st;
  return cpa::launch_prefill(a, dtype == CPA_BF16, d, stream) == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}

}  // extern "C"

namespace {
// The fused entry points: argument checks shared with the table-based calls, then one launch
// (or the split launches) with the masks in place of the tables.  bits: mask_bits / mask_words
// instead of the byte masks.
cpa_status prefill_fused(const void* q, cpa_dtype dtype, const void* k_pages, int64_t page_stride,
                         int64_t head_stride, int64_t token_stride, const void* v_pages, int v_dim_major,
                         int64_t v_page_stride, int64_t v_head_stride, int64_t v_row_stride, cpa_dtype kv_dtype,
                         float k_scale, float v_scale, int64_t n_pages,
                         const int32_t* page_map, int page_map_stride, const uint8_t* masks,
                         const uint64_t* mask_bits, bool bits, int nqb_max, int nkvb_max, int mask_words,
                         const int32_t* cu_q, const int32_t* prefix_len, int B, int Hq, int Hkv, int d,
                         int max_chunk_len, float sm_scale, void* o, float* lse, int total_q, int split_pages,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (v_dim_major != 0 && v_dim_major != 1) return CPA_ERR_SHAPE;
  if (kv_dtype != CPA_BF16 && kv_dtype != CPA_FP8_E4M3) return CPA_ERR_UNSUPPORTED;
  const bool fp8 = kv_dtype == CPA_FP8_E4M3;
  if (fp8 && (!(k_scale > 0.f) || !(v_scale > 0.f) || std::isinf(k_scale) || std::isinf(v_scale)))
    return CPA_ERR_SHAPE;
  if (nqb_max < 0 || nkvb_max < 0 || nkvb_max > CPA_MAX_KV_BLOCKS) return CPA_ERR_SHAPE;
  if (bits && (mask_words < 0 || mask_words < (nkvb_max + 63) / 64)) return CPA_ERR_SHAPE;
  if (split_pages > 0 && total_q < 0) return CPA_ERR_SHAPE;
  cpa::PrefillArgs a;
  bool nothing;
  const VLayout vl{v_page_stride, v_head_stride, v_row_stride, v_dim_major == 1};
  const cpa_status st = prepare_prefill(q, dtype, k_pages, v_pages, page_stride, head_stride, token_stride, vl,
                                        n_pages, page_map, page_map_stride, nullptr, 0, nullptr, cu_q, prefix_len,
                                        B, Hq, Hkv, d, max_chunk_len, sm_scale, o, lse, a, &nothing,
                                        /*kv_elem_bytes=*/fp8 ? 1 : 0, /*with_tables=*/false);
  if (st != CPA_OK || nothing) return st;
  const bool need = nqb_max > 0 && nkvb_max > 0;   // there are mask entries to read
  if (bits ? (need && !mask_bits) : (need && !masks)) return CPA_ERR_NULL;
  if (bits && ((uintptr_t)mask_bits & 7u) != 0) return CPA_ERR_ALIGN;
  // the direct-to-LDS bf16 kernel: 32-bit offsets within a page
  if (dtype != CPA_BF16 || token_stride > (1 << 24) || v_row_stride > (1 << 24)) return CPA_ERR_UNSUPPORTED;
  a.fused = 1;
  if (fp8) {   // as cpa_chunked_prefill_fp8kv: the K scale joins the softmax scale, the V scale the output
    a.kv_fp8 = 1;
    a.scale_log2 *= k_scale;
    a.out_scale = v_scale;
  }
  a.mask_nqb = nqb_max;
  a.mask_nkvb = nkvb_max;
  if (bits) {   // a NULL mask_bits (nothing to read) runs the byte path, which then reads nothing
    a.mask_bits = reinterpret_cast<const unsigned long long*>(mask_bits);
    a.mask_words = mask_words;
  } else {
    a.masks = masks;
    a.mask_vec = (nkvb_max % 16 == 0 && aligned16(masks)) ? 1 : 0;
  }
  if (split_pages > 0)   // a group's table holds at most nkvb_max ids
    return launch_split(a, dtype, token_stride, vl, nkvb_max, Hq, d, o, lse, total_q, split_pages, workspace,
                        workspace_bytes, stream);
  return cpa::launch_prefill(a, true, d, stream) == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}
}  // namespace

extern "C" cpa_status cpa_chunked_prefill_fused(
    const void* q, cpa_dtype dtype, const void* k_pages, int64_t page_stride, int64_t head_stride,
    int64_t token_stride, const void* v_pages, int v_dim_major, int64_t v_page_stride, int64_t v_head_stride,
    int64_t v_row_stride, cpa_dtype kv_dtype, float k_scale, float v_scale, int64_t n_pages, const int32_t* page_map,
    int page_map_stride, const uint8_t* masks, int nqb_max, int nkvb_max, const int32_t* cu_q,
    const int32_t* prefix_len, int B, int Hq, int Hkv, int d, int max_chunk_len, float sm_scale, void* o, float* lse,
    int total_q, int split_pages, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return prefill_fused(q, dtype, k_pages, page_stride, head_stride, token_stride, v_pages, v_dim_major,
                       v_page_stride, v_head_stride, v_row_stride, kv_dtype, k_scale, v_scale, n_pages, page_map,
                       page_map_stride, masks, nullptr,
                       false, nqb_max, nkvb_max, 0, cu_q, prefix_len, B, Hq, Hkv, d, max_chunk_len, sm_scale, o, lse,
                       total_q, split_pages, workspace, workspace_bytes, stream);
}

extern "C" cpa_status cpa_chunked_prefill_fused_bits(
    const void* q, cpa_dtype dtype, const void* k_pages, int64_t page_stride, int64_t head_stride,
    int64_t token_stride, const void* v_pages, int v_dim_major, int64_t v_page_stride, int64_t v_head_stride,
    int64_t v_row_stride, cpa_dtype kv_dtype, float k_scale, float v_scale, int64_t n_pages, const int32_t* page_map,
    int page_map_stride, const uint64_t* mask_bits, int nqb_max, int nkvb_max, int mask_words, const int32_t* cu_q,
    const int32_t* prefix_len, int B, int Hq, int Hkv, int d, int max_chunk_len, float sm_scale, void* o, float* lse,
    int total_q, int split_pages, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return prefill_fused(q, dtype, k_pages, page_stride, head_stride, token_stride, v_pages, v_dim_major,
                       v_page_stride, v_head_stride, v_row_stride, kv_dtype, k_scale, v_scale, n_pages, page_map,
                       page_map_stride, nullptr,
                       mask_bits, true, nqb_max, nkvb_max, mask_words, cu_q, prefix_len, B, Hq, Hkv, d,
                       max_chunk_len, sm_scale, o, lse, total_q, split_pages, workspace, workspace_bytes, stream);
}

// ---- split-KV without a caller workspace ---------------------------------------------------
// cpa_chunked_prefill_split_static keeps the split partials in `scratch`, a device array of
// CPA_STATIC_SCRATCH_BYTES that every GPU the library runs on holds until the process ends.  In
// host code the array's name is only a host-side handle, never a device address: its address
// on a device is looked up once per device, with that device current, and only that address
// is handed to the kernels.
namespace {

static __device__ __align__(256) unsigned char scratch[CPA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `device`'s copy of scratch (nullptr if the lookup fails).
void* scratch_address(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_addr[device] == nullptr) {
    int current = -1;
    if (hipGetDevice(&current) != hipSuccess) return nullptr;
    if (current != device && hipSetDevice(device) != hipSuccess) return nullptr;
    void* addr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    const hipError_t r = current != device ? hipSetDevice(current) : hipSuccess;   // restore the caller's device
    if (e != hipSuccess || r != hipSuccess || addr == nullptr) return nullptr;
    g_scratch_addr[device] = addr;
  }
  return g_scratch_addr[device];
}

}  // namespace

extern "C" cpa_status cpa_chunked_prefill_split_static(
    const void* q, cpa_dtype dtype, const void* k_pages, const void* v_pages, int64_t page_stride,
    int64_t head_stride, int64_t token_stride, int64_t n_pages, const int32_t* page_map, int page_map_stride,
    const int32_t* tables, int table_cap, const int32_t* counts, const int32_t* cu_q, const int32_t* prefix_len,
    int B, int Hq, int Hkv, int d, int max_chunk_len, float sm_scale, void* o, float* lse, int total_q,
    int split_pages, hipStream_t stream) {
  if (split_pages <= 0 || total_q < 0) return CPA_ERR_SHAPE;
  // the partials must fit the array; checked before anything touches the device
  if (cpa_split_workspace_bytes(total_q, Hq, d, table_cap, split_pages) > (size_t)CPA_STATIC_SCRATCH_BYTES)
    return CPA_ERR_CAPACITY;
  const VLayout vl{page_stride, head_stride, token_stride, false};
  cpa::PrefillArgs a;
  bool nothing;
  const cpa_status st = prepare_prefill(q, dtype, k_pages, v_pages, page_stride, head_stride, token_stride, vl,
                                        n_pages, page_map, page_map_stride, tables, table_cap, counts, cu_q,
                                        prefix_len, B, Hq, Hkv, d, max_chunk_len, sm_scale, o, lse, a, &nothing);
  if (st != CPA_OK || nothing) return st;
  int device = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &device) != hipSuccess) return CPA_ERR_LAUNCH;
  } else if (hipGetDevice(&device) != hipSuccess) {
    return CPA_ERR_LAUNCH;
  }
  void* ws = scratch_address(device);
  if (ws == nullptr) return CPA_ERR_LAUNCH;
  return prefill_split(q, dtype, k_pages, v_pages, page_stride, head_stride, token_stride, vl, n_pages, page_map,
                       page_map_stride, tables, table_cap, counts, cu_q, prefix_len, B, Hq, Hkv, d, max_chunk_len,
                       sm_scale, o, lse, total_q, split_pages, ws, (size_t)CPA_STATIC_SCRATCH_BYTES, stream);
}
