// Per-(head, query block) KV block plans: the direct block-sparse execution the union replaces.
//
// "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract:
// the method argues that executing every head's mask directly as a block-sparse kernel pays off
// poorly in chunked prefill, where a chunk holds only a few query blocks, and builds the union
// tables instead.  To measure that trade on the same hardware, this kernel builds the plans such
// a direct kernel runs: for every (sequence b, query head h, query block qi) the KV blocks kb
// its own mask row selects, with kb <= prefix_blocks[b] + qi (causally reachable), in ascending
// order, -1 after the last.
//
// One wave per mask row.  Lane l reads 16 mask bytes (16 KV blocks) per step, turns them into
// 16 bits, and the wave's prefix sum over the lanes' bit counts places every lane's ids.
#include "cpa_internal.h"

namespace cpa {
namespace {

constexpr int PT = 256;   // threads per workgroup (4 rows)

__device__ __forceinline__ uint32_t nonzero_bytes4(uint32_t x) {
  return (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
}

template <bool VEC>
__global__ __launch_bounds__(PT) void block_plan_kernel(const PlanArgs a) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * (PT / 64) + (threadIdx.x >> 6);
  const long long n_rows = (long long)a.B * a.Hq * a.nqb_max;
  if (row >= n_rows) return;
  const int qi = (int)(row % a.nqb_max);
  const int b = (int)(row / ((long long)a.Hq * a.nqb_max));
  int qb0 = min(max(a.prefix_blocks[b], 0), a.nkvb_max);
  int nqb = min(max(a.chunk_blocks[b], 0), a.nqb_max);
  nqb = min(nqb, a.nkvb_max - qb0);
  const int lim = qi < nqb ? qb0 + qi + 1 : 0;   // blocks [0, lim) are causally reachable
  const uint8_t* mrow = a.masks + (size_t)row * a.nkvb_max;
  int32_t* out = a.plans + (size_t)row * a.plan_cap;

  int base = 0;   // ids written so far
  for (int c0 = 0; c0 < lim; c0 += 64 * 16) {
    const int kb0 = c0 + 16 * lane;
    uint32_t bits = 0;
    if (kb0 < lim) {
      uint32_t v[4];
      if (VEC) {
        const uint4 x = *reinterpret_cast<const uint4*>(mrow + kb0);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t word = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int j = 4 * w + k;
            if (kb0 + j < a.nkvb_max) word |= (uint32_t)mrow[kb0 + j] << (8 * k);
          }
          v[w] = word;
        }
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t t = nonzero_bytes4(v[w]);
        bits |= ((t >> 7) & 1u) << (4 * w + 0);
        bits |= ((t >> 15) & 1u) << (4 * w + 1);
        bits |= ((t >> 23) & 1u) << (4 * w + 2);
        bits |= ((t >> 31) & 1u) << (4 * w + 3);
      }
      const int keep = lim - kb0;   // blocks kb0 .. kb0 + keep - 1 are reachable
      if (keep < 16) bits &= (1u << keep) - 1u;
    }
    // exclusive prefix sum of the lanes' counts
    const int cnt = __popc(bits);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int pos = base + incl - cnt;
    while (bits) {
      const int j = __builtin_ctz(bits);
      bits &= bits - 1u;
      out[pos++] = kb0 + j;
    }
    base += __shfl(incl, 63);
  }
  for (int i = base + lane; i < a.plan_cap; i += 64) out[i] = -1;
  if (lane == 0) a.plan_counts[row] = base;
}

}  // namespace

hipError_t launch_block_plans(const PlanArgs& a, hipStream_t s) {
  const long long n_rows = (long long)a.B * a.Hq * a.nqb_max;
  if (n_rows == 0) return hipSuccess;
  const long long n_wg = (n_rows + PT / 64 - 1) / (PT / 64);
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidValue;
  const bool vec = (a.nkvb_max % 16 == 0) && ((uintptr_t)a.masks % 16 == 0);
  if (vec)
    hipLaunchKernelGGL((block_plan_kernel<true>), dim3((unsigned)n_wg), dim3(PT), 0, s, a);
  else
    hipLaunchKernelGGL((block_plan_kernel<false>), dim3((unsigned)n_wg), dim3(PT), 0, s, a);
  return hipGetLastError();
}

}  // namespace cpa
