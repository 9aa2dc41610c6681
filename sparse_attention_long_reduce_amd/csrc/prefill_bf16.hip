// Chunked-prefill attention over per-group KV block tables for bf16 inputs, reading K/V in place
// from a paged cache (gfx950 / CDNA4).
//
// "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract:
// every query head of a GQA group attends over exactly the KV blocks of the group's table,
// which are accessed where they lie in the paged cache, with no KV compaction.
//
// Work decomposition.  A workgroup is 8 waves and owns one KV group g of one sequence b and one
// tile of query blocks.  With G = Hq/Hkv query heads per group, a wave holds one query head x
// 32 chunk rows; two waves cover the 64 rows of a query block.  For G = 4 the workgroup is the
// group's four heads on one query block; G = 2 (1) packs 2 (4) query blocks; G > 4 splits the
// heads over G/4 workgroups.  Every selected KV page is brought into LDS once per workgroup
// and read by all eight waves, i.e. by every head and row of the tile.  Two waves share each
// SIMD, so one wave's MFMAs can overlap the other's softmax.
//
// Page staging.  Each page (64 tokens x d, K and V) is copied HBM -> LDS by the gfx950
// direct-to-LDS loads (global_load_lds_dwordx4): every instruction moves 64 16-byte chunks,
// one per lane, into 1 KiB of LDS, and each lane fetches whichever chunk belongs at its LDS
// slot.  That makes the LDS layouts free to choose:
//   K: chunk c of token row r is stored at chunk c ^ swz_k(r), so the 16 rows read together by
//      one 16-byte MFMA-operand load hit 16 different bank groups;
//   V: natural [token][d] rows with chunk c at c ^ swz_v(r); the PV operand (8 consecutive
//      keys of one column per lane) is produced by two ds_read_b64_tr_b16 transposed reads,
//      which the swizzle keeps free of bank conflicts.
// No staging registers and no LDS stores are needed.  Pages are processed two per barrier and
// double-buffered in statically distinct LDS arrays (the loop is unrolled over the two buffer
// sets), so the compiler can tell the tiles being read from the ones being filled and never
// waits for the prefetch early.  The page ids of the table are resolved a window at a time
// into LDS.
//
// Per page (64 keys) and wave (32 query rows), in the transposed domain so that each lane owns
// whole query rows:
//   S^T[key][row] = K . Q^T     v_mfma_f32_32x32x16_bf16, A = K from LDS, B = Q^T in registers
//   causal cut (only when the page reaches past the wave's first row position)
//   online softmax in fp32, log2 domain, softmax scale folded into one FMA; a row's 64 scores
//   live in lanes l and l^32 (one permlane32 swap per row maximum).  The output is rescaled
//   only when a row maximum grows by more than 2^8 over the reference it was accumulated with.
//   The row sum adds the bf16-rounded weights that enter the PV product (v_dot2_f32_bf16 with
//   ones, two weights per instruction), so the result is normalised by exactly the weights used.
//   This file is compiled without NaN semantics so that maxima need no operand quieting; NaN
//   inputs still propagate through the exponentials and the MFMAs to the output.
//   O^T[dv][row] += V^T . P^T   A = V^T by transposed LDS reads, B = P^T rounded to bf16
//                               straight from the score accumulators
#include "prefill_common.h"

namespace cpa {
namespace {

constexpr int THREADS = 512;
constexpr int WIN = 1024;  // page ids resolved per window

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int D>
struct Geo {
  static constexpr int CPR = D / 8;     // 16-byte chunks per token row
  static constexpr int PAGE = 64 * D;   // bf16 elements of one K (or V) page
  static constexpr int NPW = CPR / 4;   // direct-to-LDS instructions per wave per page and tensor
  static constexpr int DT = D / 32;     // 32-wide output column tiles
};

// chunk position of K chunk c of row r is c ^ swz_k(r); of V chunk c is c ^ swz_v(r)
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// 16-byte direct-to-LDS copy: each lane's chunk at gsrc lands at ldst + 16 * lane
__device__ __forceinline__ void lds_dma16(const __bf16* gsrc, __bf16* ldst) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)ldst, 16, 0, 0);
}

__device__ __forceinline__ v4i16 ds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) char*)(__attribute__((address_space(3))) void*)p));
}

template <int D>
__global__ __launch_bounds__(THREADS) void prefill_bf16_kernel(const PrefillArgs a) {
  using GE = Geo<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 kA0[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 vA0[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 kA1[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 vA1[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 kB0[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 vB0[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 kB1[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 vB1[GE::PAGE];
  __shared__ int win_kb[WIN];
  __shared__ int win_ph[WIN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;  // lane half

  int gi, rank;
  if (!decode_tile(a, lane, gi, rank)) return;
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
  const int half = wave & 1;       // which 32 rows of the query block
  const int pair = wave >> 1;      // (head, query block) pair of this wave
  const int qi_w = qi_first + pair / a.hpw;
  const int head = g * a.G + hsub * a.hpw + (pair % a.hpw);
  const bool active = qi_w < nqb;
  const int qi_last = min(qi_first + a.qpw - 1, nqb - 1);

  const int cnt = min(max(a.counts[gi], 0), a.table_cap);
  const int32_t* tab = a.tables + (size_t)gi * a.table_cap;
  const int n_iter = cnt - count_above(tab, cnt, nqb, qb0 + qi_last, lane);
  const int n_vis = active ? cnt - count_above(tab, cnt, nqb, qb0 + qi_w, lane) : 0;

  const __bf16* __restrict__ kg = reinterpret_cast<const __bf16*>(a.k) + (size_t)g * a.head_stride;
  const __bf16* __restrict__ vg = reinterpret_cast<const __bf16*>(a.v) + (size_t)g * a.head_stride;
  const int32_t* __restrict__ pmap = a.page_map + (size_t)b * a.page_map_stride;
  const int ts = (int)a.token_stride;

  // ---- Q in registers (B operand of S^T = K Q^T) -------------------------------------------
  const int row0 = 64 * qi_w + 32 * half;   // first chunk row of this wave
  const int row = row0 + l32;               // this lane's chunk row
  const bool row_ok = active && row < Cn;
  const __bf16* qsrc = reinterpret_cast<const __bf16*>(a.q) + ((size_t)(q0 + (row_ok ? row : 0)) * a.Hq + head) * D;
  bf16x8 qb[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qsrc + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);
    qb[ks] = __builtin_bit_cast(bf16x8, u);
  }

  // ---- direct-to-LDS plan ------------------------------------------------------------------
  // waves 0-3 move K, waves 4-7 move V; wave w's instruction j fills LDS chunks
  // [(4w' + j) * 64, +64) of its tensor (w' = w % 4), lane l the chunk at position +l.
  const bool vrole = wave >= 4;
  int dma_off[GE::NPW];   // element offset of the lane's source chunk within a page
  int dma_row[GE::NPW];
#pragma unroll
  for (int j = 0; j < GE::NPW; ++j) {
    const int p = ((wave & 3) * GE::NPW + j) * 64 + lane;
    const int r = p / GE::CPR;
    const int c = (p % GE::CPR) ^ (vrole ? swz_v<D>(r) : swz_k<D>(r));
    dma_row[j] = r;
    dma_off[j] = r * ts + c * 8;
  }
  const int dma_dst = (wave & 3) * GE::NPW * 64 * 8;  // elements; + j * 512

  // A page fill is planned once and then issued one direct-to-LDS instruction at a time in
  // between the MFMAs of the QK product, so that the vector-memory queue drains while the matrix
  // core works instead of stalling the issuing wave.  Pages that are unresolved (NaN) or end
  // inside the sequence (rows past the end read as 0) are filled at once through registers.
  struct Fill {
    bool on;             // direct-to-LDS instructions still to issue
    const __bf16* src;   // this wave's tensor (K or V) of the page
    __bf16* dst;         // this wave's part of the destination tile
  };
  auto plan = [&](int kb, int ph, __bf16* ks, __bf16* vs) __attribute__((always_inline)) {
    const int nv_tok = min(max(L - 64 * kb, 0), 64);
    const __bf16* src = (vrole ? vg : kg) + (size_t)(ph < 0 ? 0 : ph) * a.page_stride;
    __bf16* dst = (vrole ? vs : ks) + dma_dst;
    Fill f{ph >= 0 && nv_tok == 64, src, dst};
    if (!f.on) {
      const uint32_t fv = ph < 0 ? 0x7FC07FC0u : 0u;
#pragma unroll
      for (int j = 0; j < GE::NPW; ++j) {
        uint4 v = make_uint4(fv, fv, fv, fv);
        if (ph >= 0 && dma_row[j] < nv_tok) v = *reinterpret_cast<const uint4*>(src + dma_off[j]);
        *reinterpret_cast<uint4*>(dst + j * 512 + lane * 8) = v;
      }
    }
    return f;
  };
  auto fill_one = [&](const Fill& f, int j) __attribute__((always_inline)) {
    if (f.on) lds_dma16(f.src + dma_off[j], f.dst + j * 512);
  };
  const Fill no_fill{false, nullptr, nullptr};

  auto load_window = [&](int base) __attribute__((always_inline)) {
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

  // ---- per-lane LDS read offsets (elements) ---------------------------------------------------
  // K operand: row l32 (+32 for keys 32-63), logical chunk 2*ks + hl
  const int k_row_off = l32 * D;
  const int k_sw = swz_k<D>(l32);
  // V operand by transposed reads: source lane s = lane % 16 points at row +(s / 4), columns
  // 32*dt + 16*((lane / 16) & 1) + 4*(s % 4) .. +3
  const int s16 = lane & 15;
  const int e_src = s16 >> 2, t4 = s16 & 3;
  const int v_row_off = (4 * hl + e_src) * D;
  const int v_sw = swz_v<D>(4 * hl + e_src);
  const int v_lo = 2 * ((lane >> 4) & 1) + (t4 >> 1);   // chunk within the 32-column tile
  const int v_in = 4 * (t4 & 1);                         // element within the chunk
  int v_off[GE::DT];
#pragma unroll
  for (int dt = 0; dt < GE::DT; ++dt) v_off[dt] = v_row_off + (((4 * dt + v_lo) ^ v_sw) << 3) + v_in;

  // ---- running softmax state and output accumulators ------------------------------------
  const float cs = a.scale_log2;
  const bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
  float m_run = -INFINITY;   // reference maximum (log2 domain) the accumulators are scaled to
  float l_run = 0.f;         // this lane's share of the row sum
  f32x16 o[GE::DT];
#pragma unroll
  for (int dt = 0; dt < GE::DT; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[dt][j] = 0.f;
  const int row_pos = P + row;
  const int wave_pos0 = P + row0;

  f32x16 s0, s1;  // S^T of the page in flight, keys 0-31 and 32-63

  // S^T = K Q^T for the page in LDS tile Kl, issuing the fill f along the way
  auto qk = [&](const __bf16* Kl, const Fill& f) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 16; ++j) { s0[j] = 0.f; s1[j] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int off = k_row_off + (((2 * ks + hl) ^ k_sw) << 3);
      const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(Kl + off);
      const bf16x8 ka1 = *reinterpret_cast<const bf16x8*>(Kl + off + 32 * D);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0, qb[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qb[ks], s1, 0, 0, 0);
      if (ks % ((D / 16) / GE::NPW) == 0) fill_one(f, ks / ((D / 16) / GE::NPW));
    }
  };
  auto fill_all = [&](const Fill& f) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < GE::NPW; ++j) fill_one(f, j);
  };

  // causal cut, online softmax and O^T += V^T P^T for page kb (scores in s0/s1, V tile Vl)
  auto softmax_pv = [&](const __bf16* Vl, int kb) __attribute__((always_inline)) {
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
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, fmaxf(s0[j], s1[j]));
    mx = xhalf_max(mx) * cs;
    const bool need = mx > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < GE::DT; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;
      m_run = m_new;
    }
    const float ref = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      s0[j] = __builtin_amdgcn_exp2f(fmaf(s0[j], cs, -ref));
      s1[j] = __builtin_amdgcn_exp2f(fmaf(s1[j], cs, -ref));
    }

    // O^T += V^T P^T; keys of step (kt, u) for lane half hl, element e:
    //   32*kt + 16*u + 8*(e / 4) + 4*hl + e % 4
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)(kt == 0 ? s0[8 * u + e] : s1[8 * u + e]);
        // the row sum accumulates the same bf16 weights the PV product uses, two per dot2
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pp = {pb[e], pb[e + 1]};
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, l_run, false);
        }
        const int krow = (32 * kt + 16 * u) * D;
#pragma unroll
        for (int dt = 0; dt < GE::DT; ++dt) {
          const v4i16 lo = ds_read_tr(Vl + krow + v_off[dt]);
          const v4i16 hi = ds_read_tr(Vl + krow + 8 * D + v_off[dt]);
          const v4i16 both[2] = {lo, hi};
          const bf16x8 va = __builtin_bit_cast(bf16x8, both);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[dt], 0, 0, 0);
        }
      }
    }
  };

  // ---- main loop ---------------------------------------------------------------------------
  // Pages go two per iteration.  Tile set A holds pages 2j and 2j+1 while set B receives pages
  // 2j+2 and 2j+3 (and the other way round on the next iteration); the loop is unrolled over
  // the two sets so that every LDS read names its tile and the compiler never has to wait for an
  // unrelated prefetch.  The page ids an iteration prefetches were read from the window one
  // iteration earlier, so no LDS latency sits in front of the prefetch.  One barrier per two
  // pages.
  if (n_iter > 0) {
    load_window(0);
    __syncthreads();
    int kb0 = win_kb[0], ph0 = win_ph[0];
    int kb1 = n_iter > 1 ? win_kb[1] : 0, ph1 = n_iter > 1 ? win_ph[1] : 0;
    fill_all(plan(kb0, ph0, kA0, vA0));
    if (n_iter > 1) fill_all(plan(kb1, ph1, kA1, vA1));
    // ids of the next pair
    int kb2 = n_iter > 2 ? win_kb[2] : 0, ph2 = n_iter > 2 ? win_ph[2] : 0;
    int kb3 = n_iter > 3 ? win_kb[3] : 0, ph3 = n_iter > 3 ? win_ph[3] : 0;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's LDS fills have landed
    __syncthreads();

    // pages p and p+1 sit in (ck0, cv0) and (ck1, cv1); pages p+2, p+3 go to (nk0, nv0), (nk1, nv1)
    auto pair = [&](int p, const __bf16* ck0, const __bf16* cv0, const __bf16* ck1, const __bf16* cv1,
                    __bf16* nk0, __bf16* nv0, __bf16* nk1, __bf16* nv1) __attribute__((always_inline)) {
      const Fill f0 = p + 2 < n_iter ? plan(kb2, ph2, nk0, nv0) : no_fill;
      const Fill f1 = p + 3 < n_iter ? plan(kb3, ph3, nk1, nv1) : no_fill;
      const int kc0 = kb0, kc1 = kb1;
      kb0 = kb2; kb1 = kb3;
      if (p + 4 < n_iter) {
        if ((p + 4) % WIN == 0) {
          load_window(p + 4);
          __syncthreads();
        }
        kb2 = win_kb[(p + 4) % WIN];
        ph2 = win_ph[(p + 4) % WIN];
        if (p + 5 < n_iter) {
          kb3 = win_kb[(p + 5) % WIN];
          ph3 = win_ph[(p + 5) % WIN];
        }
      }
      if (p < n_vis) {
        qk(ck0, f0);
        softmax_pv(cv0, kc0);
      } else {
        fill_all(f0);
      }
      if (p + 1 < n_vis) {
        qk(ck1, f1);
        softmax_pv(cv1, kc1);
      } else {
        fill_all(f1);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    };
    for (int p = 0; p < n_iter; p += 4) {
      pair(p, kA0, vA0, kA1, vA1, kB0, vB0, kB1, vB1);
      if (p + 2 < n_iter) pair(p + 2, kB0, vB0, kB1, vB1, kA0, vA0, kA1, vA1);
    }
  }

  // ---- epilogue ----------------------------------------------------------------------------
  if (!row_ok) return;
  const float lt = xhalf_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  __bf16* dst = reinterpret_cast<__bf16*>(a.o) + ((size_t)(q0 + row) * a.Hq + head) * D;
#pragma unroll
  for (int dt = 0; dt < GE::DT; ++dt) {
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

template <int D>
hipError_t launch_bf16(const PrefillArgs& a, hipStream_t s) {
  const int grid = prefill_grid(a);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_bf16_kernel<D>), dim3(grid), dim3(THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int d, hipStream_t s) {
  if (!bf16) return launch_prefill_regstaged(a, false, d, s);
  if (a.token_stride > (1 << 24)) return launch_prefill_regstaged(a, true, d, s);  // 32-bit offsets
  return d == 64 ? launch_bf16<64>(a, s) : launch_bf16<128>(a, s);
}

}  // namespace cpa
