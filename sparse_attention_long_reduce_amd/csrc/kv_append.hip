// KV append: write a prefill chunk's K and V rows into their pages of the paged cache.
//
// "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract:
// chunked prefill attends from each chunk over KV blocks that live in a paged cache and are
// read in place.  The chunk's own K/V must be in that cache first; this is the step that puts
// them there.  Row r of sequence b's chunk is token position p = prefix_len[b] + r, which lives
// in logical block p / 64, i.e. physical page page_map[b][p / 64], at slot p % 64.
//
// One workgroup of 256 threads per (sequence, chunk page, KV group): up to 64 rows of d values.
// The chunk starts on a page boundary (prefix_len is a multiple of 64), so a chunk page maps to
// one cache page.  K (and token-major V) rows are copied 16 bytes per thread, reads and writes
// both contiguous along d.  Dim-major V goes through LDS: the 64 x d tile is read row by row
// and written as d rows of 64 tokens, 16 bytes (16 fp8, 8 bf16 or 4 fp32 tokens) per thread.  Slots
// past the chunk's end are left untouched; a page that cannot be resolved (logical block past
// page_map_stride, id outside [0, n_pages)) is skipped.  A copy: bit-exact by construction.
#include "cpa_internal.h"

#include <type_traits>

namespace cpa {
namespace {

constexpr int AT = 256;   // threads per workgroup

template <int EB, int D>   // element bytes, head dim
__global__ __launch_bounds__(AT) void kv_append_kernel(const AppendArgs a) {
  constexpr int EPC = 16 / EB;     // elements per 16-byte chunk
  constexpr int CPR = D / EPC;     // chunks per token row
  // LDS tile [64][D], 16-byte chunk c of row r at chunk slot c ^ ((r / EPC) % CPR): the second
  // pass reads one column at rows EPC apart across lanes, which then fall in distinct banks
  static_assert((CPR & (CPR - 1)) == 0, "the swizzle stays within a row");
  auto sw = [](int r) { return (r / EPC) % CPR; };
  typedef uint4 chunk_t;
  typedef typename std::conditional<EB == 1, uint8_t,
                                    typename std::conditional<EB == 2, uint16_t, uint32_t>::type>::type E;
  __shared__ __attribute__((aligned(16))) unsigned char tile_raw[64 * D * EB];

  const int n_cp = a.max_chunk_len > 0 ? (a.max_chunk_len + 63) / 64 : 0;
  const int wg = blockIdx.x;
  const int g = wg % a.Hkv;
  const int j = (wg / a.Hkv) % n_cp;
  const int b = wg / (a.Hkv * n_cp);
  const int q0 = a.cu_q[b];
  const int C = min(max(a.cu_q[b + 1] - q0, 0), a.max_chunk_len);
  const int r0 = 64 * j;
  if (r0 >= C) return;
  const int nv = min(64, C - r0);
  const int P = max(a.prefix_len[b], 0);
  const int kb = (P >> 6) + j;
  if (kb >= a.page_map_stride) return;
  const int ph = a.page_map[(size_t)b * a.page_map_stride + kb];
  if (ph < 0 || (int64_t)ph >= a.n_pages) return;

  const int tid = threadIdx.x;
  const char* ksrc = static_cast<const char*>(a.k_new);
  const char* vsrc = static_cast<const char*>(a.v_new);
  char* kdst = static_cast<char*>(a.k_pages) + ((size_t)ph * a.page_stride + (size_t)g * a.head_stride) * EB;
  char* vdst = static_cast<char*>(a.v_pages) + ((size_t)ph * a.v_page_stride + (size_t)g * a.v_head_stride) * EB;
  // source row of chunk row r, head g: [Tq][Hkv][d] contiguous
  auto src_off = [&](int r) { return (((size_t)(q0 + r) * a.Hkv + g) * D) * EB; };

  for (int i = tid; i < 64 * CPR; i += AT) {
    const int r = i / CPR, c = i % CPR;
    if (r >= nv) break;
    const size_t so = src_off(r0 + r) + (size_t)c * 16;
    const int slot = r;   // r0 is a multiple of 64 and so is P
    const chunk_t kv = *reinterpret_cast<const chunk_t*>(ksrc + so);
    *reinterpret_cast<chunk_t*>(kdst + ((size_t)slot * a.token_stride + c * EPC) * EB) = kv;
    const chunk_t vv = *reinterpret_cast<const chunk_t*>(vsrc + so);
    if (!a.v_dmajor) {
      *reinterpret_cast<chunk_t*>(vdst + ((size_t)slot * a.v_row_stride + c * EPC) * EB) = vv;
    } else {
      *reinterpret_cast<chunk_t*>(tile_raw + ((size_t)r * D + (c ^ sw(r)) * EPC) * EB) = vv;
    }
  }
  if (!a.v_dmajor) return;
  __syncthreads();
  // d rows of 64 slots; 16 bytes = EPC consecutive slots per thread
  constexpr int SPR = 64 / EPC;   // chunks per dim row
  for (int i = tid; i < D * SPR; i += AT) {
    const int x = i / SPR, s0 = (i % SPR) * EPC;
    if (s0 >= nv) continue;
    unsigned char* row = reinterpret_cast<unsigned char*>(vdst) + ((size_t)x * a.v_row_stride + s0) * EB;
    // element x of row t: chunk slot (x / EPC) ^ sw(t), element x % EPC
    auto at = [&](int t) { return reinterpret_cast<const E*>(tile_raw)[t * D + (((x / EPC) ^ sw(t)) * EPC) + x % EPC]; };
    if (s0 + EPC <= nv) {
      E buf[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) buf[e] = at(s0 + e);
      *reinterpret_cast<chunk_t*>(row) = __builtin_bit_cast(chunk_t, buf);
    } else {   // the chunk's last, partial page: only the slots it owns
      for (int e = 0; s0 + e < nv; ++e) reinterpret_cast<E*>(row)[e] = at(s0 + e);
    }
  }
}

template <int EB, int D>
hipError_t launch_t(const AppendArgs& a, hipStream_t s) {
  const long long n = (long long)a.B * ((a.max_chunk_len + 63) / 64) * a.Hkv;
  if (n == 0) return hipSuccess;
  if (n > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kv_append_kernel<EB, D>), dim3((unsigned)n), dim3(AT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, int elem_bytes, int d, hipStream_t s) {
  if (elem_bytes == 1) return d == 64 ? launch_t<1, 64>(a, s) : launch_t<1, 128>(a, s);
  if (elem_bytes == 2) return d == 64 ? launch_t<2, 64>(a, s) : launch_t<2, 128>(a, s);
  return d == 64 ? launch_t<4, 64>(a, s) : launch_t<4, 128>(a, s);
}

}  // namespace cpa
