// Block-Union KV Selection: per-head 2D block masks -> per-KV-group block tables.
//
// "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract:
// the masks are KV-selection signals; a union over the chunk's query blocks and over the
// query heads of one GQA group yields the minimal per-group KV block table that keeps every
// selected block.  The table holds logical KV-block ids in ascending order.
//
// One workgroup of 1024 threads per (sequence, KV group).
//   phase 1  OR-reduce the group's G * nqb mask rows, 16 KV blocks (one 16-byte load) per
//            thread and row, four rows' loads in flight per thread, with the causal clip
//            kb <= prefix_blocks + qi applied per row; a thread walks its rows (head, query
//            block) by stepping, with no division per row;
//            partial ORs of threads that share a column meet in LDS (a tree over the row
//            splits); each 16-block column becomes 16 bits of a 64-bit word in LDS
//            (union_byte_rows, shared with the fused prefill).
//            Bit-packed masks (one bit per KV block, 64 blocks per 8-byte word) are
//            OR-reduced a word at a time instead.
//   phase 2  popcount per word, exclusive scan over words (within waves, then over the wave
//            totals), then each wave expands words: lane l of the wave owning word w writes
//            64w + l at (word offset + mbcnt rank) when bit l is set.  Positions
//            count .. table_cap-1 get -1.
// The result is unique (a set in ascending order), so the kernel is bit-exact by construction.
#include "union_common.h"

namespace cpa {
namespace {

constexpr int UT = 1024;              // threads per workgroup
constexpr int MAX_WORDS = 65536 / 64;  // 64-bit words for the largest supported KV extent

// Phase 2 for one (sequence, KV group), called by every thread of the workgroup: the
// group's nwords 64-bit words (in LDS) -> ascending ids of their set bits at tab[0 .. total),
// -1 up to table_cap, and *count = total.  Popcount per word, an exclusive scan over words
// (within waves by shuffles, then over the wave totals), then each wave expands words: lane l
// of the wave owning word w writes 64w + l at (the word's offset + its mbcnt rank) when bit l
// is set.  wpre [MAX_WORDS] and tsum [2 * UT / 64] are LDS scratch.
__device__ __forceinline__ void expand_words(const unsigned long long* words, int nwords, int32_t* tab,
                                             int table_cap, int32_t* count, int* wpre, int* tsum) {
  const int tid = threadIdx.x;
  constexpr int WPT = MAX_WORDS / UT;  // words per thread in the scan
  int pc[WPT];
  int mine = 0;
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int w = tid * WPT + k;
    pc[k] = (w < nwords) ? __popcll(words[w]) : 0;
    mine += pc[k];
  }
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) tsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int v = lane < UT / 64 ? tsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < UT / 64; off <<= 1) {
      const int y = __shfl_up(v, off);
      if (lane >= off) v += y;
    }
    if (lane < UT / 64) tsum[UT / 64 + lane] = v;   // inclusive wave prefixes
  }
  __syncthreads();
  int run = (wave > 0 ? tsum[UT / 64 + wave - 1] : 0) + incl - mine;
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int w = tid * WPT + k;
    if (w < nwords) wpre[w] = run;
    run += pc[k];
  }
  const int total = tsum[UT / 64 + UT / 64 - 1];
  __syncthreads();
  for (int w = wave; w < nwords; w += UT / 64) {
    const unsigned long long word = words[w];
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(word >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)word, 0u));
    if ((word >> lane) & 1ull) tab[wpre[w] + (int)rank] = (w << 6) + lane;
  }
  for (int i = total + tid; i < table_cap; i += UT) tab[i] = -1;
  if (tid == 0) *count = total;
}

// VEC: byte masks read 16 bytes at a time; BITS: bit-packed masks (a.mask_bits)
template <bool VEC, bool BITS>
__global__ __launch_bounds__(UT) void block_union_kernel(const UnionArgs a) {
  __shared__ unsigned long long words[MAX_WORDS];
  __shared__ uint4 red[UT];
  __shared__ int wpre[MAX_WORDS];
  __shared__ int tsum[UT];

  const int tid = threadIdx.x;
  const int b = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  const int G = a.Hq / a.Hkv;

  // clamp device-side lengths so that every access stays inside the buffers
  int qb0 = a.prefix_blocks[b];
  int nqb = a.chunk_blocks[b];
  qb0 = min(max(qb0, 0), a.nkvb_max);
  nqb = min(max(nqb, 0), a.nqb_max);
  nqb = min(nqb, a.nkvb_max - qb0);
  const int nkvb = qb0 + nqb;
  const int nwords = (nkvb + 63) >> 6;

  for (int w = tid; w < nwords; w += UT) words[w] = 0ull;
  __syncthreads();

  // ---- phase 1: OR over (head in group, query block), causal clip per row -----------------
  if (BITS) {   // union_bit_rows (union_common.h)
    const unsigned long long* wbase =
        a.mask_bits + ((size_t)b * a.Hq + (size_t)g * G) * a.nqb_max * (size_t)a.mask_words;
    union_bit_rows<UT, 4>(wbase, (size_t)a.mask_words, a.nqb_max, G, qb0, nqb, words,
                          reinterpret_cast<unsigned long long*>(red));
  } else {   // union_byte_rows (union_common.h)
    const uint8_t* gbase = a.masks + ((size_t)b * a.Hq + (size_t)g * G) * a.nqb_max * (size_t)a.nkvb_max;
    union_byte_rows<UT, 4, VEC>(gbase, (size_t)a.nkvb_max, a.nqb_max, G, qb0, nqb, a.nkvb_max, words, red);
  }

  // ---- phase 2 ------------------------------------------------------------------------------
  expand_words(words, nwords, a.tables + ((size_t)b * a.Hkv + g) * a.table_cap, a.table_cap,
               a.counts + (size_t)b * a.Hkv + g, wpre, tsum);
}

}  // namespace

hipError_t launch_block_union(const UnionArgs& a, hipStream_t s) {
  if (a.B == 0 || a.Hkv == 0) return hipSuccess;
  const bool vec = (a.nkvb_max % 16 == 0) && ((uintptr_t)a.masks % 16 == 0);
  dim3 grid((unsigned)(a.B * a.Hkv)), block(UT);
  if (a.use_bits) {
    hipLaunchKernelGGL((block_union_kernel<false, true>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  if (vec)
    hipLaunchKernelGGL((block_union_kernel<true, false>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((block_union_kernel<false, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace cpa
