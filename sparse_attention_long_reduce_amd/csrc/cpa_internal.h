// Internal launch interface shared by the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpa {

// (query block, head) pairs per prefill workgroup: one pair per two waves (64 query rows)
constexpr int PAIRS_PER_TILE = 4;

// 64-bit words of a per-group block bitmap at the largest supported KV extent (65536 blocks)
constexpr int MAX_KV_WORDS = 65536 / 64;

struct UnionArgs {
  const uint8_t* masks;
  int B, Hq, Hkv, nqb_max, nkvb_max;
  const int32_t* prefix_blocks;
  const int32_t* chunk_blocks;
  int32_t* tables;
  int table_cap;
  int32_t* counts;
  // bit-packed masks instead of bytes (masks unused): row (b, h, qi) is mask_words 64-bit words,
  // bit kb % 64 of word kb / 64 = block kb selected
  const unsigned long long* mask_bits;
  int mask_words;
  int use_bits;   // 1: read mask_bits (may be NULL only when there is no mask row to read)
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t page_stride, head_stride, token_stride, n_pages;  // elements / pages (K; V unless below)
  // V pool: element (page, group, token, dim) at page * v_page_stride + group * v_head_stride +
  // token * v_row_stride + dim (v_dmajor == 0, token-major pages) or + dim * v_row_stride + token
  // (v_dmajor == 1, dim-major pages)
  int64_t v_page_stride, v_head_stride, v_row_stride;
  int v_dmajor;
  // fp8 KV: the pools hold OCP e4m3 bytes (strides in elements = bytes) of values x * k_scale and
  // x * v_scale; the K scale is folded into scale_log2 and the V scale is out_scale
  int kv_fp8;
  float out_scale;      // multiplies the normalised output (1 unless fp8 KV)
  const int32_t* page_map;
  int page_map_stride;
  const int32_t* tables;
  int table_cap;
  const int32_t* counts;
  const int32_t* cu_q;
  const int32_t* prefix_len;
  int B, Hq, Hkv, max_chunk_len;
  float scale_log2;  // softmax scale * log2(e)
  void* o;
  float* lse;
  // work decomposition (filled by the launcher)
  int G;                // query heads per KV group
  // A KV group's (query block, head) pairs, numbered qi * G + h, are cut into tiles of
  // PAIRS_PER_TILE consecutive pairs (see tile_pairs in prefill_common.h)
  int tiles_per_group;  // ceil(max query blocks * G / PAIRS_PER_TILE)
  int n_groups;         // B * Hkv
  int xcd_remap;        // 1: keep each KV group's tiles on one XCD (see the prefill kernel)
  // split-KV: the pages each tile visits are cut into n_splits near-equal ranges (at most
  // split_pages each); range s of a tile writes its rows' normalised partial output (fp32
  // part_o[s][row][head][d]) and LSE (part_lse[s][row][head], natural log) instead of o / lse.
  // n_splits == 1: no split.
  int n_splits;
  int split_pages;
  int total_q;          // rows of all sequences (the partials' row dimension)
  float* part_o;
  float* part_lse;
  // fused block union (fused == 1): no tables / counts; every workgroup ORs its KV group's
  // rows of masks (uint8 [B][Hq][mask_nqb][mask_nkvb], nonzero = selected) itself, with
  // prefix_blocks = prefix_len / 64 and chunk_blocks = the chunk's query blocks.  mask_vec: rows
  // can be read 16 bytes at a time (mask_nkvb % 16 == 0 and a 16-byte aligned base).
  int fused;
  const uint8_t* masks;
  int mask_nqb, mask_nkvb, mask_vec;
  // fused from bit-packed masks (masks unused): uint64 [B][Hq][mask_nqb][mask_words], bit kb % 64
  // of word kb / 64 = block kb selected
  const unsigned long long* mask_bits;
  int mask_words;
};

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  int n_splits, total_q, Hq;
  void* o;       // bf16 [total_q][Hq][d]
  float* lse;    // optional [total_q][Hq]
};

// KV append: rows [Tq][Hkv][d] of k_new / v_new go to their slots of the paged pools (layouts
// as in PrefillArgs)
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_pages;
  void* v_pages;
  int64_t page_stride, head_stride, token_stride, n_pages;
  int64_t v_page_stride, v_head_stride, v_row_stride;
  int v_dmajor;
  const int32_t* page_map;
  int page_map_stride;
  const int32_t* cu_q;
  const int32_t* prefix_len;
  int B, Hkv, max_chunk_len;
};

// per-(head, query block) plans of the direct block-sparse baseline
struct PlanArgs {
  const uint8_t* masks;   // [B][Hq][nqb_max][nkvb_max]
  int B, Hq, nqb_max, nkvb_max;
  const int32_t* prefix_blocks;
  const int32_t* chunk_blocks;
  int32_t* plans;         // [B][Hq][nqb_max][plan_cap]
  int plan_cap;
  int32_t* plan_counts;   // [B][Hq][nqb_max]
};

// direct block-sparse prefill (bf16, dim-major V): every wave runs one (head, query block, half)
// over its own plan, operands loaded from memory straight into registers
struct DirectArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t page_stride, head_stride, token_stride;          // K, token-major
  int64_t v_page_stride, v_head_stride, v_dim_stride;      // V, dim-major
  int64_t n_pages;
  const int32_t* page_map;
  int page_map_stride;
  const int32_t* plans;
  int plan_cap;
  const int32_t* plan_counts;
  const int32_t* cu_q;
  const int32_t* prefix_len;
  int B, Hq, Hkv, max_chunk_len, nqb_max;
  float scale_log2;
  void* o;
  float* lse;
  int xcd_remap;
};

// All return hipSuccess or the launch error; they never synchronise.
hipError_t launch_block_union(const UnionArgs& a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int d, hipStream_t s);
// combines the split-KV partials (bf16 output)
hipError_t launch_split_merge(const MergeArgs& m, int d, hipStream_t s);
// register-staged variant (V transposed through registers); serves fp32 and is kept for bf16
// as the reference point of the direct-to-LDS bf16 kernel
hipError_t launch_prefill_regstaged(const PrefillArgs& a, bool bf16, int d, hipStream_t s);
hipError_t launch_kv_append(const AppendArgs& a, int elem_bytes, int d, hipStream_t s);
hipError_t launch_block_plans(const PlanArgs& a, hipStream_t s);
hipError_t launch_prefill_direct(const DirectArgs& a, int d, hipStream_t s);

}  // namespace cpa
