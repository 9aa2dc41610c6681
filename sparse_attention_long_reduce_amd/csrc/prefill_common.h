// Device helpers shared by the prefill kernels.
#pragma once
#include "cpa_internal.h"
#include <climits>

namespace cpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
// log2 headroom before the output accumulators must be rescaled to a new row maximum
constexpr float kRescaleThreshold = 8.0f;

// a lane's 16 weights of one unit may sum to this before the row reference must move (2^30)
constexpr float kSumLimit = 1073741824.0f;

// Key order of K operand rows when V operands are 8 consecutive keys (dim-major V).  The score
// accumulator of lane l holds, in elements 0..7, rows 4(l/32) + 0..3 and 8 + 4(l/32) + 0..3 of
// each 16-row half, and those elements become the lane's 8 k-values of the PV product's P
// operand.  Loading K row m from key key_perm(m) (bits 2 and 3 swapped) puts exactly the keys
// 8(l/32) + 0..7 in those elements, matching the V operand.
__device__ __forceinline__ int key_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// 8 e4m3 codes (OCP fp8) -> their 8 values in bf16 (exact), as one 16-byte chunk; each
// instruction converts the two codes of the low (false) or high (true) 16 bits, scale 1
__device__ __forceinline__ uint4 fp8x8_to_bf16(uint2 x) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t h[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, false),
                         __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, true),
                         __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, false),
                         __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, true)};
  return __builtin_bit_cast(uint4, h);
}

// max / sum of x over lanes l and l^32 (the two lanes that share a query row)
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Number of the last `nqb` table entries (the only ones that can lie past a query block of the
// chunk when the table is ascending) whose id exceeds `lim`; wave-uniform.
__device__ __forceinline__ int count_above(const int32_t* tab, int cnt, int nqb, int lim, int lane) {
  int c = 0;
  for (int base = max(0, cnt - nqb); base < cnt; base += 64) {
    const int i = base + lane;
    const int v = (i < cnt) ? tab[i] : INT_MIN;
    c += __popcll(__builtin_amdgcn_ballot_w64(v > lim));
  }
  return c;
}

// Pages KV group gi's tiles are expected to visit: its table length, or with FU (no table
// yet) the sequence's causal extent in blocks, the bound of its table length.
template <bool FU>
__device__ __forceinline__ int group_weight(const PrefillArgs& a, int gi) {
  if (FU) {
    const int b = gi / a.Hkv;
    const int cn = min(max(a.cu_q[b + 1] - a.cu_q[b], 0), a.max_chunk_len);
    return (max(a.prefix_len[b], 0) >> 6) + ((cn + 63) >> 6);
  }
  return min(max(a.counts[gi], 0), a.table_cap);
}

// Position of lane j's KV group (j < ngx, the groups gi = xcd + 8*j) when the groups of one XCD
// are sorted by group_weight, heaviest first (ties by j); wave-uniform loop over ngx <= 64.
template <bool FU>
__device__ __forceinline__ int weight_rank(const PrefillArgs& a, int xcd, int ngx, int lane) {
  const int c = lane < ngx ? group_weight<FU>(a, xcd + 8 * lane) : -1;
  int r = 0;
  for (int i = 0; i < ngx; ++i) {
    const int ci = __shfl(c, i);
    r += (ci > c) || (ci == c && i < lane);
  }
  return r;
}

// Workgroup -> (KV group index gi = b*Hkv + g, tile rank, split).  Workgroups are dispatched
// round-robin over the 8 XCDs (blockIdx % 8) and, within an XCD, in blockIdx order as CUs free
// up.  With xcd_remap every tile of one KV group lands on the same XCD, so the group's pages
// are shared through that XCD's L2.  Work is handed out longest first: the groups of an XCD in
// decreasing table length (a tile visits about as many pages as its group's table holds), and
// within a group the tiles of rank 0 (the last query blocks, which see the most pages) first,
// the split ranges of one tile next to each other.  Beyond 64 groups per XCD the groups go in
// index order.  Returns false for padding.  FU: the tables are built by the workgroups
// themselves, so groups are ordered by their causal extent instead.
template <bool FU>
__device__ __forceinline__ bool decode_tile(const PrefillArgs& a, int lane, int& gi, int& rank, int& split) {
  const int per_group = a.tiles_per_group * a.n_splits;   // work items of one KV group
  int w;
  if (a.xcd_remap) {
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int ngx = (a.n_groups - xcd + 7) >> 3;  // groups gi with gi % 8 == xcd
    if (slot >= ngx * per_group) return false;
    int k = slot / per_group;
    w = slot - k * per_group;
    if (ngx <= 64) {
      const uint64_t hit = __builtin_amdgcn_ballot_w64(weight_rank<FU>(a, xcd, ngx, lane) == k);
      k = __builtin_ctzll(hit);
    }
    gi = xcd + 8 * k;
  } else {
    if ((int)blockIdx.x >= a.n_groups * per_group) return false;
    gi = blockIdx.x % a.n_groups;
    w = blockIdx.x / a.n_groups;
  }
  rank = w / a.n_splits;
  split = w - rank * a.n_splits;
  return true;
}

// Pairs of tile t of a KV group with G query heads.  The group's (query block qi, head h) pairs
// are numbered qi * G + h and tile t holds pairs 4t .. 4t+3, so every group size fills the
// workgroup's four pair slots (a tile may span two or more query blocks).  For wave pair slot
// `slot`: qi_w / h_w are that pair's query block and head within the group; qi_first / qi_last are
// the first and last query block the tile touches (before clamping to the chunk).
__device__ __forceinline__ void tile_pairs(int t, int slot, int G, int& qi_first, int& qi_last, int& qi_w, int& h_w) {
  const int p0 = PAIRS_PER_TILE * t;
  qi_first = p0 / G;
  qi_last = (p0 + PAIRS_PER_TILE - 1) / G;
  const int p = p0 + slot;
  qi_w = p / G;
  h_w = p - qi_w * G;
}

inline int prefill_grid(const PrefillArgs& a) {
  const int per_group = a.tiles_per_group * a.n_splits;
  return a.xcd_remap ? 8 * ((a.n_groups + 7) / 8) * per_group : a.n_groups * per_group;
}

}  // namespace cpa
