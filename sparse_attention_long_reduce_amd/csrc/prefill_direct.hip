// Direct block-sparse chunked prefill: the baseline the union tables are measured against.
//
// "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract:
// executing every head's block mask directly pays off poorly when a chunk holds only a few query
// blocks, which is the method's reason for the union tables: they trade extra blocks for page
// reuse across a group's heads and query blocks.  This kernel is that direct execution on the same
// hardware and numerics: every (sequence, query head, query block) attends over exactly the KV
// blocks of its own plan (cpa_build_block_plans), with no union and no page shared between
// heads or query blocks.
//
// Since no page is shared, staging pages in LDS would buy nothing: a wave (32 query rows of one
// head) loads its MFMA operands straight from memory into registers, 16 bytes per lane, and
// needs no LDS and no barrier.  That needs the V operand (8 consecutive keys of one column) to
// be one 16-byte chunk, i.e. dim-major V pages; the K slab rows are then taken in the key_perm
// order of the union kernel so that the score accumulators hand PV those same keys.  A
// workgroup is the two waves (64 rows) of one (head, query block); the tiles of a KV group go
// to one XCD, last query blocks first.  Numerics as in the union kernel: Q pre-scaled by
// scale*log2(e) in bf16, bf16 MFMA with fp32 accumulation, weights against a lazily moved row
// reference, bf16 P, row sums over the bf16 weights.
#include "prefill_common.h"

namespace cpa {
namespace {

constexpr int DTH = 128;   // threads per workgroup

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int D>
__global__ __launch_bounds__(DTH, 2) void prefill_direct_kernel(const DirectArgs a) {
  constexpr int KS = D / 16;   // k-steps of QK
  constexpr int DT = D / 32;   // 32-wide output column tiles
  const int lane = threadIdx.x & 63;
  const int half = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int G = a.Hq / a.Hkv;
  const int per_group = G * a.nqb_max;
  const int n_groups = a.B * a.Hkv;

  int gi, t;
  if (a.xcd_remap) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int k = slot / per_group;
    gi = xcd + 8 * k;
    t = slot - k * per_group;
    if (gi >= n_groups) return;
  } else {
    gi = blockIdx.x % n_groups;
    t = blockIdx.x / n_groups;
    if (t >= per_group) return;
  }
  const int b = gi / a.Hkv, g = gi - b * a.Hkv;
  const int qi = a.nqb_max - 1 - t / G;      // heaviest (last) query blocks first
  const int head = g * G + t % G;

  const int P = max(a.prefix_len[b], 0);
  const int q0 = a.cu_q[b];
  const int Cn = min(max(a.cu_q[b + 1] - q0, 0), a.max_chunk_len);
  if (64 * qi >= Cn) return;   // uniform over the workgroup
  const int L = P + Cn;
  const int row0 = 64 * qi + 32 * half;
  const int row = row0 + l32;
  const bool row_ok = row < Cn;
  const int row_pos = P + row;
  const int wave_pos0 = P + row0;

  const size_t prow = ((size_t)b * a.Hq + head) * a.nqb_max + qi;
  const int n = min(max(a.plan_counts[prow], 0), a.plan_cap);
  const int32_t* plan = a.plans + prow * a.plan_cap;
  const int32_t* pmap = a.page_map + (size_t)b * a.page_map_stride;
  const __bf16* kg = reinterpret_cast<const __bf16*>(a.k) + (size_t)g * a.head_stride;
  const __bf16* vg = reinterpret_cast<const __bf16*>(a.v) + (size_t)g * a.v_head_stride;
  const size_t ts = (size_t)a.token_stride, vds = (size_t)a.v_dim_stride;

  // Q (B operand of S^T = K Q^T), pre-scaled into log2 units
  const __bf16* qsrc = reinterpret_cast<const __bf16*>(a.q) + ((size_t)(q0 + (row_ok ? row : 0)) * a.Hq + head) * D;
  bf16x8 qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qsrc + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);
    const bf16x8 raw = __builtin_bit_cast(bf16x8, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[ks][e] = (__bf16)((float)raw[e] * a.scale_log2);
  }

  // operand loads of unit u = (plan entry u / 2, key half u % 2)
  const bf16x8 nan8 = __builtin_bit_cast(bf16x8, make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u));
  const int krow_lane = key_perm(l32);
  auto page_of = [&](int i, int& kb, int& ph) __attribute__((always_inline)) {
    kb = plan[i];
    ph = -1;
    if (kb >= 0 && kb < a.page_map_stride) {
      ph = pmap[kb];
      if (ph < 0 || (int64_t)ph >= a.n_pages) ph = -1;
    }
  };
  auto load_k = [&](int ph, int hh, bf16x8* ka) __attribute__((always_inline)) {
    if (ph < 0) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[ks] = nan8;
      return;
    }
    const __bf16* src = kg + (size_t)ph * a.page_stride + (size_t)(32 * hh + krow_lane) * ts + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
  };
  auto load_v = [&](int kb, int ph, int hh, bf16x8 (*va)[DT]) __attribute__((always_inline)) {
    const int key0 = 64 * kb + 32 * hh + 8 * hl;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if (ph < 0) {
          va[u][dt] = nan8;
          continue;
        }
        bf16x8 x = *reinterpret_cast<const bf16x8*>(vg + (size_t)ph * a.v_page_stride +
                                                    (size_t)(32 * dt + l32) * vds + 32 * hh + 16 * u + 8 * hl);
        const int k0 = key0 + 16 * u;
        if (k0 + 8 > L) {   // keys past the sequence end (the last, partial page): zero
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k0 + e >= L) x[e] = (__bf16)0.0f;
        }
        va[u][dt] = x;
      }
  };

  const bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
  float m_run = 0.f, l_run = 0.f;
  f32x16 cm;
#pragma unroll
  for (int j = 0; j < 16; ++j) cm[j] = 0.f;
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[dt][j] = 0.f;

  auto rowmax = [&](const f32x16& s) __attribute__((always_inline)) {
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int j = 3; j < 15; j += 2) mx = fmaxf(fmaxf(mx, s[j]), s[j + 1]);
    return xhalf_max(fmaxf(mx, s[15]));
  };
  auto weights = [&](const f32x16& s, bf16x8& p0, bf16x8& p1) __attribute__((always_inline)) {
    float w[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = __builtin_amdgcn_exp2f(s[j]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p0[e] = (__bf16)w[e];
      p1[e] = (__bf16)w[8 + e];
    }
    float lu = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      lu = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[e], p0[e + 1]}, kOnes2, lu, false);
      lu = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[e], p1[e + 1]}, kOnes2, lu, false);
    }
    return lu;
  };

  const int n_units = 2 * n;
  int kb_n = 0, ph_n = -1;
  bf16x8 kn[KS];
  if (n_units > 0) {
    page_of(0, kb_n, ph_n);
    load_k(ph_n, 0, kn);
  }
  for (int u = 0; u < n_units; ++u) {
    const int hh = u & 1;
    const int kb = kb_n, ph = ph_n;
    bf16x8 ka[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = kn[ks];
    if (u + 1 < n_units) {   // K of the next unit in flight during this one
      if (hh == 1) page_of((u + 1) >> 1, kb_n, ph_n);
      load_k(ph_n, hh ^ 1, kn);
    }
    // QK against the reference (the accumulator starts at -m)
    f32x16 s;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qb[ks], ks == 0 ? cm : s, 0, 0, 0);
    // V of this unit, in flight during the softmax (its registers reuse those of K)
    bf16x8 va[2][DT];
    load_v(kb, ph, hh, va);
    const int k0 = 64 * kb + 32 * hh;
    if (k0 + 31 > wave_pos0) {   // causal cut
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = k0 + 16 * (j >> 3) + 8 * hl + (j & 7);
        if (key > row_pos) s[j] = -INFINITY;
      }
    }
    if (u == 0) {   // the first reference: this unit's row maximum
      const float mx = rowmax(s);
      m_run = mx > -INFINITY ? mx : 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[j] -= m_run;
        cm[j] = -m_run;
      }
    }
    bf16x8 p0, p1;
    float lu = weights(s, p0, p1);
    if (__builtin_amdgcn_ballot_w64(!(lu < kSumLimit))) {   // move the reference (rare)
      const float mx = rowmax(s);
      const float d = mx > kRescaleThreshold ? mx : 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[j] -= d;
        cm[j] -= d;
      }
      m_run += d;
      const float alpha = __builtin_amdgcn_exp2f(-d);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;
      lu = weights(s, p0, p1);
    }
    l_run += lu;
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[uu][dt], uu == 0 ? p0 : p1, o[dt], 0, 0, 0);
  }

  if (!row_ok) return;
  const float lt = xhalf_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  __bf16* dst = reinterpret_cast<__bf16*>(a.o) + ((size_t)(q0 + row) * a.Hq + head) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __bf16 h4[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) h4[c] = (__bf16)(o[dt][4 * q + c] * inv);
      *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * q + 4 * hl) = __builtin_bit_cast(uint2, h4);
    }
  }
  if (a.lse != nullptr && hl == 0)
    a.lse[(size_t)(q0 + row) * a.Hq + head] = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_prefill_direct(const DirectArgs& a, int d, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const long long per_group = (long long)G * a.nqb_max;
  const long long n_groups = (long long)a.B * a.Hkv;
  const long long grid = a.xcd_remap ? 8 * ((n_groups + 7) / 8) * per_group : n_groups * per_group;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (d == 64)
    hipLaunchKernelGGL((prefill_direct_kernel<64>), dim3((unsigned)grid), dim3(DTH), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_direct_kernel<128>), dim3((unsigned)grid), dim3(DTH), 0, s, a);
  return hipGetLastError();
}

}  // namespace cpa
