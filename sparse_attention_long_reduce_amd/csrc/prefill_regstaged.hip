// Chunked-prefill attention over per-group KV block tables, reading K/V in place from a paged
// cache (gfx950 / CDNA4): register-staged variant.  It serves fp32 inputs; for bf16 the
// direct-to-LDS kernel (prefill_bf16.hip) is the production path and this one is kept as its
// point of comparison.
//
// "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract:
// every query head of a GQA group attends over exactly the KV blocks of the group's table,
// which are accessed where they lie in the paged cache, with no KV compaction.
//
// Work decomposition.  A workgroup is 8 waves and owns one KV group g of one sequence b and one
// tile of query blocks.  With G = Hq/Hkv query heads per group, a wave holds one query head x
// 32 chunk rows; two waves cover the 64 rows of a query block.  For G = 4 the workgroup is the
// group's four heads on one query block; G = 2 (1) packs 2 (4) query blocks; G > 4 splits the
// heads over G/4 workgroups.  Every selected KV page is staged into LDS once per workgroup and
// read by all eight waves, i.e. by every head and row of the tile.  Two waves share each SIMD,
// so one wave's MFMAs overlap the other's softmax.
//
// Per page (64 keys) and wave (32 query rows), computed in the transposed domain so that each
// lane owns whole query rows:
//   S^T[key][row] = K . Q^T            MFMA, A = K rows from LDS, B = Q^T held in registers
//   causal cut (only when the page reaches past the wave's first row position)
//   online softmax in fp32, log2 domain with the softmax scale folded into one FMA; a row's 64
//   scores live in lanes l and l^32 (one permlane32 swap per row maximum).  The output is only
//   rescaled when some row's maximum grows by more than 2^8 over the reference it was
//   accumulated with, so the steady state has no rescale; the final division by the row sum
//   makes the result independent of the reference.
//   O^T[dv][row] += V^T . P^T          MFMA, A = V^T from LDS, B = P^T straight from the
//                                      score accumulators (no LDS round trip)
// bf16: v_mfma_f32_32x32x16_bf16, P rounded to bf16 before the PV product.
// fp32: v_mfma_f32_32x32x2f32 end to end.
// fp8 KV (KV8, with bf16 Q): the pages hold OCP e4m3 codes, converted on their way into LDS to
// bf16, which holds every e4m3 value exactly; the per-tensor scales are applied outside the
// products (the K scale joins the softmax scale, the V scale the final normalisation), and
// everything after the staging is the bf16 path.
//
// V is written to LDS transposed ([dv][key]); in the bf16 path the key order inside each
// 32-key half is permuted (bits 2 and 3 of the key index swapped) so that the 8 keys a lane
// contributes to one PV step are contiguous and the A operand is a single 16-byte LDS read.
//
// Pipelining: pages are double-buffered in LDS.  While page i is consumed, page i+1 is loaded
// from HBM into registers (waves 0-3 load V, waves 4-7 load K; issued before the MFMAs of page
// i) and written to the other LDS buffer afterwards; one barrier per page.  Physical page ids
// are resolved a window at a time into LDS so that no dependent scalar load sits on the
// critical path.
//
// Launch order: workgroups go round-robin over the 8 XCDs (blockIdx % 8).  Tiles are mapped so
// that all tiles of one KV group run on one XCD, where they share that XCD's L2 while streaming
// the same pages in the same order; within an XCD the tiles with the most visible pages (the
// last query blocks) start first.
#include "prefill_common.h"
#include <type_traits>

namespace cpa {
namespace {

constexpr int THREADS = 512;
constexpr int ROLE = 256;          // threads per staging role (V: waves 0-3, K: waves 4-7)
constexpr int WIN = 1024;          // physical page ids resolved per window
constexpr float LN2 = kLn2;
constexpr float RESCALE_TH = kRescaleThreshold;

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

template <bool BF, int D>
struct Cfg {
  using T = typename std::conditional<BF, __bf16, float>::type;
  static constexpr int EB = BF ? 2 : 4;             // bytes per element
  static constexpr int EPC = 16 / EB;               // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;               // 16-byte chunks per token row
  static constexpr int KS = D + EPC;                // K row stride in LDS (elements; +16 B pad)
  static constexpr int VS = 64 + EPC;               // V^T row stride in LDS (elements; +16 B pad)
  static constexpr int STAGE = 64 * KS + D * VS;    // elements per LDS stage (K then V^T)
  static constexpr int KCH = 64 * CPR / ROLE;       // 16-byte K chunks per K-role thread
  static constexpr int VUNITS = 16 * CPR;           // (key quad, 16-byte column) units of V
  static constexpr int VPT = (VUNITS + ROLE - 1) / ROLE;
  static constexpr int NST = KCH > 4 * VPT ? KCH : 4 * VPT;  // staging registers (uint4)
  static constexpr int DT = D / 32;                 // 32-wide output column tiles
};

template <bool BF, int D, bool KV8>
__global__ __launch_bounds__(THREADS) void prefill_kernel(const PrefillArgs a) {
  using C = Cfg<BF, D>;
  using T = typename C::T;
  using KT = typename std::conditional<KV8, uint8_t, T>::type;   // pool element
  __shared__ __attribute__((aligned(16))) T smem[2 * C::STAGE];
  __shared__ int win_kb[WIN];
  __shared__ int win_ph[WIN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;  // lane half

  // ---- tile decode ---------------------------------------------------------------------
  int gi, rank, split;   // split-KV is not taken on this path (n_splits == 1)
  if (!decode_tile<false>(a, lane, gi, rank, split)) return;
  const int b = gi / a.Hkv;
  const int g = gi - b * a.Hkv;
  const int t_pairs = a.tiles_per_group - 1 - rank;   // heaviest (last) query blocks first

  const int P = max(a.prefix_len[b], 0);
  const int q0 = a.cu_q[b];
  const int Cn = min(max(a.cu_q[b + 1] - q0, 0), a.max_chunk_len);
  const int nqb = (Cn + 63) >> 6;
  const int half = wave & 1;       // which 32 rows of the query block
  const int pair = wave >> 1;      // (query block, head) pair slot of this wave
  int qi_first, qi_span, qi_w, h_w;
  tile_pairs(t_pairs, pair, a.G, qi_first, qi_span, qi_w, h_w);
  if (qi_first >= nqb) return;  // uniform over the workgroup
  const int qb0 = P >> 6;
  const int L = P + Cn;
  const int head = g * a.G + h_w;
  const bool active = qi_w < nqb;
  const int qi_last = min(qi_span, nqb - 1);

  const int cnt = min(max(a.counts[gi], 0), a.table_cap);
  const int32_t* tab = a.tables + (size_t)gi * a.table_cap;
  const int n_iter = cnt - count_above(tab, cnt, nqb, qb0 + qi_last, lane);
  const int n_vis = active ? cnt - count_above(tab, cnt, nqb, qb0 + qi_w, lane) : 0;

  const KT* __restrict__ kg = reinterpret_cast<const KT*>(a.k) + (size_t)g * a.head_stride;
  const KT* __restrict__ vg = reinterpret_cast<const KT*>(a.v) + (size_t)g * a.v_head_stride;
  // the 16-byte chunk of EPC elements (in the compute type) that starts at p
  auto chunk_at = [&](const KT* p) __attribute__((always_inline)) {
    if constexpr (KV8) return fp8x8_to_bf16(*reinterpret_cast<const uint2*>(p));
    else return *reinterpret_cast<const uint4*>(p);
  };
  const int32_t* __restrict__ pmap = a.page_map + (size_t)b * a.page_map_stride;
  const int64_t ts = a.token_stride;
  const int64_t vrs = a.v_row_stride;
  // 16-byte chunk `col` of V token row r of the page at vp: one load for token-major pages, a
  // gather of EPC elements (one per dim row) for dim-major pages
  auto v_chunk = [&](const KT* vp, int r, int col) __attribute__((always_inline)) {
    if (!a.v_dmajor) return chunk_at(vp + (size_t)r * vrs + col * C::EPC);
    KT e[C::EPC];
#pragma unroll
    for (int x = 0; x < C::EPC; ++x) e[x] = vp[(size_t)(col * C::EPC + x) * vrs + r];
    if constexpr (KV8) return fp8x8_to_bf16(__builtin_bit_cast(uint2, e));
    else return __builtin_bit_cast(uint4, e);
  };

  // ---- Q in registers (B operand of S^T = K Q^T) -------------------------------------------
  const int row0 = 64 * qi_w + 32 * half;   // first chunk row of this wave
  const int row = row0 + l32;               // this lane's chunk row
  const bool row_ok = active && row < Cn;
  const T* qsrc = reinterpret_cast<const T*>(a.q) + ((size_t)(q0 + (row_ok ? row : 0)) * a.Hq + head) * D;
  bf16x8 qb[BF ? D / 16 : 1];
  f32x4 qf[BF ? 1 : D / 8];
  if constexpr (BF) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qsrc + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);
      qb[ks] = __builtin_bit_cast(bf16x8, u);
    }
  } else {
#pragma unroll
    for (int kq = 0; kq < D / 8; ++kq) {
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
      if (row_ok) u = *reinterpret_cast<const f32x4*>(qsrc + hl * (D / 2) + 4 * kq);
      qf[kq] = u;
    }
  }

  // ---- staging -----------------------------------------------------------------------------
  const bool vrole = wave < 4;
  const int rtid = tid & (ROLE - 1);
  uint4 st[C::NST];

  // page (kb, ph) -> registers.  Fast path: a resolved page wholly inside the sequence.  Slow
  // path: rows at or past the sequence end read as 0; an unresolved page reads as NaN.
  auto stage_load = [&](int kb, int ph) {
    const int nv_tok = min(max(L - 64 * kb, 0), 64);
    if (ph >= 0 && nv_tok == 64) {
      if (vrole) {
        const KT* vp = vg + (size_t)ph * a.v_page_stride;
#pragma unroll
        for (int k = 0; k < C::VPT; ++k) {
          const int u = min(rtid + ROLE * k, C::VUNITS - 1);
          const int col = u % C::CPR, q4 = u / C::CPR;
#pragma unroll
          for (int c = 0; c < 4; ++c) st[4 * k + c] = v_chunk(vp, 4 * q4 + c, col);
        }
      } else {
        const KT* kp = kg + (size_t)ph * a.page_stride;
#pragma unroll
        for (int k = 0; k < C::KCH; ++k) {
          const int ch = rtid + ROLE * k;
          st[k] = chunk_at(kp + (size_t)(ch / C::CPR) * ts + (ch % C::CPR) * C::EPC);
        }
      }
    } else {
      const uint32_t f = (ph < 0) ? (BF ? 0x7FC07FC0u : 0x7FC00000u) : 0u;
      const uint4 fill = make_uint4(f, f, f, f);
      const size_t pofs = (size_t)(ph < 0 ? 0 : ph) * a.page_stride;
      if (vrole) {
        const KT* vp = vg + (size_t)(ph < 0 ? 0 : ph) * a.v_page_stride;
#pragma unroll
        for (int k = 0; k < C::VPT; ++k) {
          const int u = min(rtid + ROLE * k, C::VUNITS - 1);
          const int col = u % C::CPR, q4 = u / C::CPR;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = 4 * q4 + c;
            st[4 * k + c] = (ph >= 0 && r < nv_tok) ? v_chunk(vp, r, col) : fill;
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < C::KCH; ++k) {
          const int ch = rtid + ROLE * k;
          const int r = ch / C::CPR;
          st[k] = (ph >= 0 && r < nv_tok) ? chunk_at(kg + pofs + (size_t)r * ts + (ch % C::CPR) * C::EPC) : fill;
        }
      }
    }
  };

  auto stage_store = [&](int buf) {
    T* Kl = smem + buf * C::STAGE;
    T* Vl = Kl + 64 * C::KS;
    if (vrole) {
#pragma unroll
      for (int k = 0; k < C::VPT; ++k) {
        const int u = rtid + ROLE * k;
        if (u >= C::VUNITS) continue;
        const int col = u % C::CPR, q4 = u / C::CPR;
        const uint4 k0 = st[4 * k], k1 = st[4 * k + 1], k2 = st[4 * k + 2], k3 = st[4 * k + 3];
        if constexpr (BF) {
          // keys 4*q4 .. 4*q4+3 x 8 columns -> 8 rows of V^T, 4 keys each (8 bytes)
          const int pq = (q4 & ~3) | ((q4 & 1) << 1) | ((q4 >> 1) & 1);  // key-quad permutation
          T* dst = Vl + (col * 8) * C::VS + 4 * pq;
          const uint32_t a0[4] = {k0.x, k0.y, k0.z, k0.w}, a1[4] = {k1.x, k1.y, k1.z, k1.w};
          const uint32_t a2[4] = {k2.x, k2.y, k2.z, k2.w}, a3[4] = {k3.x, k3.y, k3.z, k3.w};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            *reinterpret_cast<uint2*>(dst + (2 * w) * C::VS) = make_uint2(pack_lo(a0[w], a1[w]), pack_lo(a2[w], a3[w]));
            *reinterpret_cast<uint2*>(dst + (2 * w + 1) * C::VS) = make_uint2(pack_hi(a0[w], a1[w]), pack_hi(a2[w], a3[w]));
          }
        } else {
          // keys 4*q4 .. 4*q4+3 x 4 columns -> 4 rows of V^T, 4 keys each (16 bytes)
          T* dst = Vl + (col * 4) * C::VS + 4 * q4;
          *reinterpret_cast<uint4*>(dst + 0 * C::VS) = make_uint4(k0.x, k1.x, k2.x, k3.x);
          *reinterpret_cast<uint4*>(dst + 1 * C::VS) = make_uint4(k0.y, k1.y, k2.y, k3.y);
          *reinterpret_cast<uint4*>(dst + 2 * C::VS) = make_uint4(k0.z, k1.z, k2.z, k3.z);
          *reinterpret_cast<uint4*>(dst + 3 * C::VS) = make_uint4(k0.w, k1.w, k2.w, k3.w);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < C::KCH; ++k) {
        const int ch = rtid + ROLE * k;
        *reinterpret_cast<uint4*>(Kl + (ch / C::CPR) * C::KS + (ch % C::CPR) * C::EPC) = st[k];
      }
    }
  };

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

  // ---- running softmax state and output accumulators ------------------------------------
  const float cs = a.scale_log2;
  float m_run = -INFINITY;   // reference maximum (log2 domain) the accumulators are scaled to
  float l_run = 0.f;         // this lane's share of the row sum
  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[dt][j] = 0.f;
  const int row_pos = P + row;                 // absolute position of this lane's row
  const int wave_pos0 = P + row0;              // of the wave's first row

  auto compute_page = [&](int buf, int kb) {
    const T* Kl = smem + buf * C::STAGE;
    const T* Vl = Kl + 64 * C::KS;
    f32x16 s0, s1;  // S^T for keys 0-31 and 32-63 of the page
#pragma unroll
    for (int j = 0; j < 16; ++j) { s0[j] = 0.f; s1[j] = 0.f; }

    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(Kl + l32 * C::KS + 16 * ks + 8 * hl);
        const bf16x8 ka1 = *reinterpret_cast<const bf16x8*>(Kl + (32 + l32) * C::KS + 16 * ks + 8 * hl);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0, qb[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qb[ks], s1, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kq = 0; kq < D / 8; ++kq) {
        const f32x4 ka0 = *reinterpret_cast<const f32x4*>(Kl + l32 * C::KS + hl * (D / 2) + 4 * kq);
        const f32x4 ka1 = *reinterpret_cast<const f32x4*>(Kl + (32 + l32) * C::KS + hl * (D / 2) + 4 * kq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(ka0[e], qf[kq][e], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(ka1[e], qf[kq][e], s1, 0, 0, 0);
        }
      }
    }

    // causal cut: key position 64*kb + key index must not exceed the row position
    if (64 * kb + 63 > wave_pos0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = 64 * kb + 8 * (j >> 2) + 4 * hl + (j & 3);
        if (key > row_pos) s0[j] = -INFINITY;
        if (key + 32 > row_pos) s1[j] = -INFINITY;
      }
    }

    // online softmax (log2 domain), lazy rescale
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fmaxf(s0[j], s1[j]));
    mx = xhalf_max(mx) * cs;
    const bool need = mx > m_run + RESCALE_TH;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;
      m_run = m_new;
    }
    const float ref = (m_run == -INFINITY) ? 0.f : m_run;
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      s0[j] = __builtin_amdgcn_exp2f(fmaf(s0[j], cs, -ref));
      s1[j] = __builtin_amdgcn_exp2f(fmaf(s1[j], cs, -ref));
      sum += s0[j] + s1[j];
    }
    l_run += sum;

    // O^T += V^T P^T
    if constexpr (BF) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = (__bf16)(kt == 0 ? s0[8 * u + e] : s1[8 * u + e]);
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) {
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vl + (32 * dt + l32) * C::VS + 32 * kt + 16 * u + 8 * hl);
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[dt], 0, 0, 0);
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
              o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[c], kt == 0 ? s0[4 * q + c] : s1[4 * q + c], o[dt], 0, 0, 0);
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
  if (!row_ok) return;
  const float lt = xhalf_sum(l_run);
  const float inv = lt > 0.f ? a.out_scale / lt : 0.f;
  T* dst = reinterpret_cast<T*>(a.o) + ((size_t)(q0 + row) * a.Hq + head) * D;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int dv = 32 * dt + 8 * q + 4 * hl;
      if constexpr (BF) {
        __bf16 h4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) h4[c] = (__bf16)(o[dt][4 * q + c] * inv);
        *reinterpret_cast<uint2*>(dst + dv) = __builtin_bit_cast(uint2, h4);
      } else {
        f32x4 v4;
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = o[dt][4 * q + c] * inv;
        *reinterpret_cast<f32x4*>(dst + dv) = v4;
      }
    }
  }
  if (a.lse != nullptr && hl == 0)
    a.lse[(size_t)(q0 + row) * a.Hq + head] = lt > 0.f ? (m_run + __log2f(lt)) * LN2 : -INFINITY;   // scores include the K scale
}

template <bool BF, int D, bool KV8 = false>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
  const int grid = prefill_grid(a);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_kernel<BF, D, KV8>), dim3(grid), dim3(THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_regstaged(const PrefillArgs& a, bool bf16, int d, hipStream_t s) {
  if (a.kv_fp8) return d == 64 ? launch_t<true, 64, true>(a, s) : launch_t<true, 128, true>(a, s);
  if (bf16) return d == 64 ? launch_t<true, 64>(a, s) : launch_t<true, 128>(a, s);
  return d == 64 ? launch_t<false, 64>(a, s) : launch_t<false, 128>(a, s);
}

}  // namespace cpa
