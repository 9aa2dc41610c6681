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
//            kb <= prefix_blocks + qi applied per row;
//            partial ORs of threads that share a column meet in LDS (a tree over the row
//            splits); each 16-block column becomes 16 bits of a 64-bit word in LDS.
//            Bit-packed masks (one bit per KV block, 64 blocks per 8-byte word) are
//            OR-reduced a word at a time instead.
//   phase 2  popcount per word, exclusive scan over words (within waves, then over the wave
//            totals), then each wave expands words: lane l of the wave owning word w writes
//            64w + l at (word offset + mbcnt rank) when bit l is set.  Positions
//            count .. table_cap-1 get -1.
// The result is unique (a set in ascending order), so the kernel is bit-exact by construction.
#include "cpa_internal.h"

namespace cpa {
namespace {

constexpr int UT = 1024;              // threads per workgroup
constexpr int MAX_WORDS = 65536 / 64;  // 64-bit words for the largest supported KV extent

// 0x80 in every byte of x that is nonzero
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
  return (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
}

// 16 mask bytes -> 16 bits (bit j set iff byte j nonzero)
__device__ __forceinline__ uint32_t bytes_to_bits(const uint32_t v[4]) {
  uint32_t bits = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t t = nonzero_bytes(v[w]);
    bits |= ((t >> 7) & 1u) << (4 * w + 0);
    bits |= ((t >> 15) & 1u) << (4 * w + 1);
    bits |= ((t >> 23) & 1u) << (4 * w + 2);
    bits |= ((t >> 31) & 1u) << (4 * w + 3);
  }
  return bits;
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
  if (BITS) {
    // column c = word c (KV blocks 64c .. 64c+63); row t as in the byte path below
    int lgw = 0;
    while ((1 << lgw) < nwords && (1 << lgw) < UT) ++lgw;
    const int colw = 1 << lgw;
    const int rs = UT >> lgw;
    const size_t wstride = (size_t)a.mask_words;
    const unsigned long long* wbase =
        a.mask_bits + ((size_t)b * a.Hq + (size_t)g * G) * a.nqb_max * wstride;
    unsigned long long* redw = reinterpret_cast<unsigned long long*>(red);
    for (int c0 = 0; c0 < nwords; c0 += colw) {
      const int c = c0 + (tid & (colw - 1));
      const int s = tid >> lgw;
      unsigned long long acc = 0ull;
      if (c < nwords) {
        const int kb0 = c << 6;
        const int qi_lo = max(0, kb0 - qb0);
        const int nq = nqb - qi_lo;
        const int nrows = G * nq;
        auto row = [&](int t) __attribute__((always_inline)) {
          const int hh = t / nq;
          const int qi = qi_lo + (t - hh * nq);
          unsigned long long v = wbase[((size_t)hh * a.nqb_max + qi) * wstride + c];
          const int nallow = qb0 + qi - kb0 + 1;   // bits 0 .. nallow-1 are causally reachable
          if (nallow < 64) v &= (1ull << nallow) - 1ull;   // nallow >= 1 here (qi >= qi_lo)
          return v;
        };
        for (int t0 = s; t0 < nrows; t0 += 4 * rs) {
          unsigned long long v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int t = t0 + u * rs;
            v[u] = t < nrows ? row(t) : 0ull;
          }
          acc |= (v[0] | v[1]) | (v[2] | v[3]);
        }
      }
      redw[tid] = acc;
      __syncthreads();
      for (int h = rs >> 1; h >= 1; h >>= 1) {   // tree OR over the row splits of a column
        if (s < h) redw[tid] |= redw[tid + (h << lgw)];
        __syncthreads();
      }
      if (s == 0 && c < nwords) words[c] = redw[tid];
      __syncthreads();
    }
  }
  const int nchunk = BITS ? 0 : (nkvb + 15) >> 4;
  int lg = 0;
  while ((1 << lg) < nchunk && (1 << lg) < UT) ++lg;
  const int cols = 1 << lg;
  const int rsplit = UT >> lg;
  const size_t row_stride = (size_t)a.nkvb_max;
  const uint8_t* gbase = a.masks + ((size_t)b * a.Hq + (size_t)g * G) * a.nqb_max * row_stride;

  for (int c0 = 0; c0 < nchunk; c0 += cols) {
    const int c = c0 + (tid & (cols - 1));
    const int s = tid >> lg;
    uint32_t acc[4] = {0u, 0u, 0u, 0u};
    if (c < nchunk) {
      const int kb0 = c << 4;
      const int qi_lo = max(0, kb0 - qb0);  // first query block that can reach column kb0
      const int nq = nqb - qi_lo;
      // mask bytes of row t (head t / nq of the group, query block qi_lo + t % nq) at column
      // kb0, causally clipped
      auto row = [&](int t, uint32_t v[4]) __attribute__((always_inline)) {
        const int hh = t / nq;
        const int qi = qi_lo + (t - hh * nq);
        const uint8_t* rowp = gbase + ((size_t)hh * a.nqb_max + qi) * row_stride + kb0;
        if (VEC) {
          const uint4 x = *reinterpret_cast<const uint4*>(rowp);
          v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else {
          const int lim = min(16, a.nkvb_max - kb0);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t word = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int j = 4 * w + k;
              if (j < lim) word |= (uint32_t)rowp[j] << (8 * k);
            }
            v[w] = word;
          }
        }
        const int nallow = qb0 + qi - kb0 + 1;  // bytes 0 .. nallow-1 are causally reachable
        if (nallow < 16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int keep = min(max(nallow - 4 * w, 0), 4);
            const uint32_t m = keep >= 4 ? 0xFFFFFFFFu : ((1u << (8 * keep)) - 1u);
            v[w] &= m;
          }
        }
      };
      const int nrows = G * nq;
      for (int t0 = s; t0 < nrows; t0 += 4 * rsplit) {
        uint32_t v[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = t0 + u * rsplit;
          if (t < nrows) {
            row(t, v[u]);
          } else {
            v[u][0] = v[u][1] = v[u][2] = v[u][3] = 0u;
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[w] |= v[u][w];
      }
    }
    red[tid] = make_uint4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    for (int h = rsplit >> 1; h >= 1; h >>= 1) {   // tree OR over the row splits of a column
      if (s < h) {
        const uint4 o = red[tid + (h << lg)];
        const uint4 m = red[tid];
        red[tid] = make_uint4(m.x | o.x, m.y | o.y, m.z | o.z, m.w | o.w);
      }
      __syncthreads();
    }
    if (s == 0 && c < nchunk) {
      const uint4 m = red[tid];
      const uint32_t v[4] = {m.x, m.y, m.z, m.w};
      reinterpret_cast<unsigned short*>(words)[c] = (unsigned short)bytes_to_bits(v);  // little endian
    }
    __syncthreads();
  }

  // ---- phase 2: popcount, exclusive scan over words, expansion ----------------------------
  constexpr int WPT = MAX_WORDS / UT;  // words per thread in the scan
  int pc[WPT];
  int mine = 0;
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int w = tid * WPT + k;
    pc[k] = (w < nwords) ? __popcll(words[w]) : 0;
    mine += pc[k];
  }
  // exclusive scan of the per-thread sums: inclusive scan within each wave, then over the
  // 16 wave totals in wave 0
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

  int32_t* tab = a.tables + ((size_t)b * a.Hkv + g) * a.table_cap;
  for (int w = wave; w < nwords; w += UT / 64) {
    const unsigned long long word = words[w];
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(word >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)word, 0u));
    if ((word >> lane) & 1ull) tab[wpre[w] + (int)rank] = (w << 6) + lane;
  }
  for (int i = total + tid; i < a.table_cap; i += UT) tab[i] = -1;
  if (tid == 0) a.counts[(size_t)b * a.Hkv + g] = total;
}

}  // namespace

hipError_t launch_block_union(const UnionArgs& a, hipStream_t s) {
  if (a.B == 0 || a.Hkv == 0) return hipSuccess;
  dim3 grid((unsigned)(a.B * a.Hkv)), block(UT);
  if (a.use_bits) {
    hipLaunchKernelGGL((block_union_kernel<false, true>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  const bool vec = (a.nkvb_max % 16 == 0) && ((uintptr_t)a.masks % 16 == 0);
  if (vec)
    hipLaunchKernelGGL((block_union_kernel<true, false>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((block_union_kernel<false, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace cpa
