// Chunked-prefill attention over per-group KV block tables, reading K/V in place from a paged
// cache (gfx950 / CDNA4).
//
// "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract:
// every query head of a GQA group attends over exactly the KV blocks of the group's table,
// which are accessed where they lie in the paged cache, with no KV compaction.
//
// Work decomposition.  A workgroup is 4 waves and owns one KV group g of one sequence b and
// one tile of query blocks: with G = Hq/Hkv query heads per group, each wave holds one query
// head x 64 chunk rows (one query block).  For G = 4 the four waves are the group's four heads
// on the same query block; G = 2 (1) packs 2 (4) query blocks; G > 4 splits the heads over
// G/4 workgroups.  Every selected KV page is staged into LDS once per workgroup and used by
// all its waves, i.e. by every head and row of the tile.
//
// Per page (64 keys) and wave (64 query rows), computed in the transposed domain so that each
// lane owns whole query rows:
//   S^T[key][row] = K . Q^T            MFMA, A = K rows from LDS, B = Q^T held in registers
//   causal cut (only when the page reaches past the wave's first row position)
//   online softmax in fp32, log2 domain with the softmax scale folded into one FMA;
//   a row's 64 scores live in lanes l and l^32 (one permlane32 swap per max)
//   O^T[dv][row] += V^T . P^T          MFMA, A = V^T from LDS, B = P^T straight from the
//                                      score accumulators (no LDS round trip)
// bf16: v_mfma_f32_32x32x16_bf16, P rounded to bf16 before the PV product.
// fp32: v_mfma_f32_32x32x2f32 end to end.
//
// V is written to LDS transposed ([dv][key]); in the bf16 path the key order inside each
// 32-key half is permuted (bits 2 and 3 of the key index swapped) so that the 8 keys a lane
// contributes to one PV step are contiguous and the A operand is a single 16-byte LDS read.
//
// Pipelining: pages are double-buffered in LDS.  While page i is consumed, page i+1 is loaded
// from HBM into registers (issued before the MFMAs of page i) and written to the other LDS
// buffer afterwards; one barrier per page.  Physical page ids are resolved a window at a time
// into LDS so that no dependent scalar load sits on the critical path.
//
// Launch order: workgroups go round-robin over the 8 XCDs (blockIdx % 8).  Tiles are mapped so
// that all tiles of one KV group run on one XCD, where they share that XCD's L2 while streaming
// the same pages in the same order; within an XCD the tiles with the most visible pages (the
// last query blocks) start first.
#include "cpa_internal.h"
#include <climits>
#include <type_traits>

namespace cpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int THREADS = 256;
constexpr int WIN = 512;  // physical page ids resolved per window
constexpr float LN2 = 0.69314718055994530942f;

__device__ __forceinline__ float xhalf_max(float x) {
  // max of x over lanes l and l^32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// number of the last `nqb` table entries (the only ones that can lie past a query block of the
// chunk when the table is ascending) whose id exceeds `lim`; wave-uniform
__device__ __forceinline__ int count_above(const int32_t* tab, int cnt, int nqb, int lim, int lane) {
  int c = 0;
  for (int base = max(0, cnt - nqb); base < cnt; base += 64) {
    const int i = base + lane;
    const int v = (i < cnt) ? tab[i] : INT_MIN;
    c += __popcll(__builtin_amdgcn_ballot_w64(v > lim));
  }
  return c;
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

template <bool BF, int D>
struct Cfg {
  using T = typename std::conditional<BF, __bf16, float>::type;
  static constexpr int EB = BF ? 2 : 4;             // bytes per element
  static constexpr int EPC = 16 / EB;               // elements per 16-byte chunk
  static constexpr int KS = D + EPC;                // K row stride in LDS (elements; +16 B pad)
  static constexpr int VS = 64 + EPC;               // V^T row stride in LDS (elements; +16 B pad)
  static constexpr int STAGE = 64 * KS + D * VS;    // elements per LDS stage (K then V^T)
  static constexpr int KCH = 64 * (D / EPC) / THREADS;  // 16-byte K chunks per thread
  static constexpr int VUNITS = 16 * (D / EPC);     // (key quad, 16-byte column) units of V
  static constexpr int VPT = (VUNITS + THREADS - 1) / THREADS;
  static constexpr int DT = D / 32;                 // 32-wide output column tiles
};

template <bool BF, int D>
__global__ __launch_bounds__(THREADS, 1) void prefill_kernel(const PrefillArgs a) {
  using C = Cfg<BF, D>;
  using T = typename C::T;
  __shared__ __attribute__((aligned(16))) T smem[2 * C::STAGE];
  __shared__ int win_kb[WIN];
  __shared__ int win_ph[WIN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;  // lane half

  // ---- tile decode ---------------------------------------------------------------------
  int gi, rank;
  if (a.xcd_remap) {
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int ngx = (a.n_groups - xcd + 7) >> 3;  // groups gi with gi % 8 == xcd
    if (slot >= ngx * a.tiles_per_group) return;
    gi = xcd + 8 * (slot % ngx);
    rank = slot / ngx;
  } else {
    if ((int)blockIdx.x >= a.n_groups * a.tiles_per_group) return;
    gi = blockIdx.x % a.n_groups;
    rank = blockIdx.x / a.n_groups;
  }
  const int b = gi / a.Hkv;
  const int g = gi - b * a.Hkv;
  const int hsub = rank % a.hsplit;
  const int qt = a.n_qtiles - 1 - rank / a.hsplit;  // heaviest (last) query blocks first

  const int P = max(a.prefix_len[b], 0);
  const int q0 = a.cu_q[b];
  const int Cn = min(max(a.cu_q[b + 1] - q0, 0), a.max_chunk_len);
  const int nqb = (Cn + 63) >> 6;
  const int qi_first = qt * a.qpw;
  if (qi_first >= nqb) return;  // uniform over the workgroup
  const int qb0 = P >> 6;
  const int L = P + Cn;
  const int qi_w = qi_first + wave / a.hpw;
  const int head = g * a.G + hsub * a.hpw + (wave % a.hpw);
  const bool active = qi_w < nqb;
  const int qi_last = min(qi_first + a.qpw - 1, nqb - 1);

  const int cnt = min(max(a.counts[gi], 0), a.table_cap);
  const int32_t* tab = a.tables + (size_t)gi * a.table_cap;
  const int n_iter = cnt - count_above(tab, cnt, nqb, qb0 + qi_last, lane);
  const int n_vis = active ? cnt - count_above(tab, cnt, nqb, qb0 + qi_w, lane) : 0;

  const T* __restrict__ kg = reinterpret_cast<const T*>(a.k) + (size_t)g * a.head_stride;
  const T* __restrict__ vg = reinterpret_cast<const T*>(a.v) + (size_t)g * a.head_stride;
  const int32_t* pmap = a.page_map + (size_t)b * a.page_map_stride;

  auto load_window = [&](int base) {
    for (int j = tid; j < WIN && base + j < n_iter; j += THREADS) {
      const int kb = tab[base + j];
      int ph = -1;
      if (kb >= 0 && kb < a.page_map_stride) {
        ph = pmap[kb];
        if (ph < 0 || (int64_t)ph >= a.n_pages) ph = -1;
      }
      win_kb[j] = kb;
      win_ph[j] = ph;
    }
  };

  // ---- Q in registers (B operand of S^T = K Q^T) -------------------------------------------
  const T* qbase = reinterpret_cast<const T*>(a.q);
  const int row_in_chunk0 = 64 * qi_w + l32;  // + 32*rt
  bf16x8 qb[2][BF ? D / 16 : 1];
  f32x4 qf[2][BF ? 1 : D / 8];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = row_in_chunk0 + 32 * rt;
    const bool ok = active && r < Cn;
    const T* src = qbase + ((size_t)(q0 + (ok ? r : 0)) * a.Hq + head) * D;
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        uint4 u = ok ? *reinterpret_cast<const uint4*>(src + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);
        qb[rt][ks] = __builtin_bit_cast(bf16x8, u);
      }
    } else {
#pragma unroll
      for (int kq = 0; kq < D / 8; ++kq) {
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
        if (ok) u = *reinterpret_cast<const f32x4*>(src + hl * (D / 2) + 4 * kq);
        qf[rt][kq] = u;
      }
    }
  }

  // ---- staging registers ---------------------------------------------------------------
  uint4 kreg[C::KCH];
  uint4 vreg[C::VPT][4];

  // load page (kb, ph) into registers; rows at or past the sequence end read as 0, pages that
  // cannot be resolved read as NaN
  auto stage_load = [&](int kb, int ph) {
    const int nv_tok = min(max(L - 64 * kb, 0), 64);
    const uint32_t fill = (ph < 0) ? (BF ? 0x7FC07FC0u : 0x7FC00000u) : 0u;
    const uint4 fill4 = make_uint4(fill, fill, fill, fill);
    const T* kp = kg + (size_t)(ph < 0 ? 0 : ph) * a.page_stride;
    const T* vp = vg + (size_t)(ph < 0 ? 0 : ph) * a.page_stride;
#pragma unroll
    for (int k = 0; k < C::KCH; ++k) {
      const int ch = tid + THREADS * k;
      const int row = ch / (D / C::EPC);
      const int col = ch % (D / C::EPC);
      kreg[k] = (ph >= 0 && row < nv_tok)
                    ? *reinterpret_cast<const uint4*>(kp + (size_t)row * a.token_stride + col * C::EPC)
                    : fill4;
    }
#pragma unroll
    for (int k = 0; k < C::VPT; ++k) {
      const int u = tid + THREADS * k;
      const int col = u % (D / C::EPC);
      const int q4 = u / (D / C::EPC);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int row = 4 * q4 + c;
        vreg[k][c] = (u < C::VUNITS && ph >= 0 && row < nv_tok)
                         ? *reinterpret_cast<const uint4*>(vp + (size_t)row * a.token_stride + col * C::EPC)
                         : fill4;
      }
    }
  };

  auto stage_store = [&](int buf) {
    T* Kl = smem + buf * C::STAGE;
    T* Vl = Kl + 64 * C::KS;
#pragma unroll
    for (int k = 0; k < C::KCH; ++k) {
      const int ch = tid + THREADS * k;
      const int row = ch / (D / C::EPC);
      const int col = ch % (D / C::EPC);
      *reinterpret_cast<uint4*>(Kl + row * C::KS + col * C::EPC) = kreg[k];
    }
#pragma unroll
    for (int k = 0; k < C::VPT; ++k) {
      const int u = tid + THREADS * k;
      if (u >= C::VUNITS) continue;
      const int col = u % (D / C::EPC);
      const int q4 = u / (D / C::EPC);
      const uint32_t* k0 = reinterpret_cast<const uint32_t*>(&vreg[k][0]);
      const uint32_t* k1 = reinterpret_cast<const uint32_t*>(&vreg[k][1]);
      const uint32_t* k2 = reinterpret_cast<const uint32_t*>(&vreg[k][2]);
      const uint32_t* k3 = reinterpret_cast<const uint32_t*>(&vreg[k][3]);
      if constexpr (BF) {
        // keys 4*q4 .. 4*q4+3 x 8 columns -> 8 rows of V^T, 4 keys each (8 bytes)
        const int pq = (q4 & ~3) | ((q4 & 1) << 1) | ((q4 >> 1) & 1);  // key-quad permutation
        T* dst = Vl + (col * 8) * C::VS + 4 * pq;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint2 lo = make_uint2(pack_lo(k0[w], k1[w]), pack_lo(k2[w], k3[w]));
          const uint2 hi = make_uint2(pack_hi(k0[w], k1[w]), pack_hi(k2[w], k3[w]));
          *reinterpret_cast<uint2*>(dst + (2 * w) * C::VS) = lo;
          *reinterpret_cast<uint2*>(dst + (2 * w + 1) * C::VS) = hi;
        }
      } else {
        // keys 4*q4 .. 4*q4+3 x 4 columns -> 4 rows of V^T, 4 keys each (16 bytes)
        T* dst = Vl + (col * 4) * C::VS + 4 * q4;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          *reinterpret_cast<uint4*>(dst + w * C::VS) = make_uint4(k0[w], k1[w], k2[w], k3[w]);
      }
    }
  };

  // ---- running softmax state and output accumulators ------------------------------------
  const float cs = a.scale_log2;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x16 o[C::DT][2];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[dt][rt][j] = 0.f;

  const int row_pos0 = P + row_in_chunk0;  // absolute position of this lane's row (rt = 0)

  auto compute_page = [&](int buf, int kb) {
    const T* Kl = smem + buf * C::STAGE;
    const T* Vl = Kl + 64 * C::KS;
    f32x16 s[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[kt][rt][j] = 0.f;

    // S^T = K Q^T
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kl + (32 * kt + l32) * C::KS + 16 * ks + 8 * hl);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            s[kt][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[rt][ks], s[kt][rt], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int kq = 0; kq < D / 8; ++kq) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const f32x4 ka = *reinterpret_cast<const f32x4*>(Kl + (32 * kt + l32) * C::KS + hl * (D / 2) + 4 * kq);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
              s[kt][rt] = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[e], qf[rt][kq][e], s[kt][rt], 0, 0, 0);
        }
      }
    }

    // causal cut: key position 64*kb + key index must not exceed the row position
    if (64 * kb + 63 > P + 64 * qi_w) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = 64 * kb + 32 * kt + 8 * (j >> 2) + 4 * hl + (j & 3);
            if (key > row_pos0 + 32 * rt) s[kt][rt][j] = -INFINITY;
          }
    }

    // online softmax (log2 domain)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kt][rt][j]);
      mx = xhalf_max(mx);
      const float m_new = fmaxf(m_run[rt], mx * cs);
      const float ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - ref);
      m_run[rt] = m_new;
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][rt][j], cs, -ref));
          s[kt][rt][j] = p;
          sum += p;
        }
      l_run[rt] = fmaf(l_run[rt], alpha, sum);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[dt][rt][j] *= alpha;
    }

    // O^T += V^T P^T
    if constexpr (BF) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          bf16x8 pb[2];
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[rt][e] = (__bf16)s[kt][rt][8 * u + e];
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) {
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vl + (32 * dt + l32) * C::VS + 32 * kt + 16 * u + 8 * hl);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
              o[dt][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[rt], o[dt][rt], 0, 0, 0);
          }
        }
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) {
            const f32x4 va = *reinterpret_cast<const f32x4*>(Vl + (32 * dt + l32) * C::VS + 32 * kt + 8 * q + 4 * hl);
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int rt = 0; rt < 2; ++rt)
                o[dt][rt] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[c], s[kt][rt][4 * q + c], o[dt][rt], 0, 0, 0);
          }
        }
      }
    }
  };

  // ---- main loop -------------------------------------------------------------------------
  if (n_iter > 0) {
    load_window(0);
    __syncthreads();
    int kb_cur = win_kb[0];
    stage_load(kb_cur, win_ph[0]);
    stage_store(0);
    __syncthreads();
    for (int i = 0; i < n_iter; ++i) {
      const bool has_next = i + 1 < n_iter;
      int kb_nx = 0;
      if (has_next) {
        if ((i + 1) % WIN == 0) {
          load_window(i + 1);
          __syncthreads();
        }
        kb_nx = win_kb[(i + 1) % WIN];
        stage_load(kb_nx, win_ph[(i + 1) % WIN]);
      }
      if (i < n_vis) compute_page(i & 1, kb_cur);
      if (has_next) stage_store((i + 1) & 1);
      __syncthreads();
      kb_cur = kb_nx;
    }
  }

  // ---- epilogue ----------------------------------------------------------------------------
  if (!active) return;
  T* obase = reinterpret_cast<T*>(a.o);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const float lt = xhalf_sum(l_run[rt]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int r = row_in_chunk0 + 32 * rt;
    if (r >= Cn) continue;
    T* dst = obase + ((size_t)(q0 + r) * a.Hq + head) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dv = 32 * dt + 8 * q + 4 * hl;
        if constexpr (BF) {
          __bf16 h4[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) h4[c] = (__bf16)(o[dt][rt][4 * q + c] * inv);
          *reinterpret_cast<uint2*>(dst + dv) = __builtin_bit_cast(uint2, h4);
        } else {
          f32x4 v4;
#pragma unroll
          for (int c = 0; c < 4; ++c) v4[c] = o[dt][rt][4 * q + c] * inv;
          *reinterpret_cast<f32x4*>(dst + dv) = v4;
        }
      }
    }
    if (a.lse != nullptr && hl == 0)
      a.lse[(size_t)(q0 + r) * a.Hq + head] = lt > 0.f ? (m_run[rt] + __log2f(lt)) * LN2 : -INFINITY;
  }
}

template <bool BF, int D>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
  const int grid = a.xcd_remap ? 8 * ((a.n_groups + 7) / 8) * a.tiles_per_group
                               : a.n_groups * a.tiles_per_group;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_kernel<BF, D>), dim3(grid), dim3(THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int d, hipStream_t s) {
  if (bf16) return d == 64 ? launch_t<true, 64>(a, s) : launch_t<true, 128>(a, s);
  return d == 64 ? launch_t<false, 64>(a, s) : launch_t<false, 128>(a, s);
}

}  // namespace cpa
