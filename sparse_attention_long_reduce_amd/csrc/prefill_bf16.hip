// Chunked-prefill attention over per-group KV block tables for bf16 inputs, reading K/V in place
// from a paged cache (gfx950 / CDNA4).
//
// "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract:
// every query head of a GQA group attends over exactly the KV blocks of the group's table,
// which are accessed where they lie in the paged cache, with no KV compaction.
//
// Work decomposition.  A workgroup is 8 waves and owns one KV group g of one sequence b and one
// tile of four (query block, head) pairs.  With G = Hq/Hkv query heads per group, the group's
// pairs are numbered qi * G + h and a tile takes four consecutive ones (tile_pairs in
// prefill_common.h); two waves cover the 64 rows of a pair, one query head x 32 chunk rows
// each.  For G = 4 a tile is the group's four heads on one query block; G = 2 (1) packs 2 (4)
// query blocks; G = 8 gives each query block two tiles; any other G fills the four slots the
// same way, a tile then spanning two query blocks.  Every selected KV page is brought into LDS
// once per workgroup and read by all eight waves, i.e. by every head and row of the tile.
//
// Page staging.  Each page (64 tokens x d, K and V) is copied HBM -> LDS by the gfx950
// direct-to-LDS loads (global_load_lds_dwordx4): every instruction moves 64 16-byte chunks,
// one per lane, into 1 KiB of LDS, and each lane fetches whichever chunk belongs at its LDS
// slot.  That makes the LDS layouts free to choose:
//   K: in MFMA operand order.  Slab (h, ks) (1 KiB) holds, at 16-byte slot l, key 32h + l % 32,
//      chunk 2ks + l / 32: the operand of lane l for k-step ks of key half h.  Every operand
//      load is then one contiguous, conflict-free 1 KiB read at an immediate offset.  With
//      dim-major V the keys of a slab are permuted (key_perm in prefill_common.h), see V below;
//   V: the PV operand of lane l is 8 consecutive keys of one output column.  A pool of
//      token-major pages ([token][d], d contiguous) is staged as natural rows with chunk c at
//      c ^ swz_v(r), and each operand is built by two ds_read_b64_tr_b16 transposed reads,
//      which the swizzle keeps free of bank conflicts.  A pool of dim-major pages ([d][token],
//      tokens contiguous) holds those 8 keys in one 16-byte chunk, so it is staged in operand
//      order like K: slab (h, u, dt) holds, at slot l, column 32dt + l % 32, keys
//      32h + 16u + 8(l / 32) .. +7, and each operand is one ds_read_b128.  The transposed read
//      delivers half the bytes per LDS cycle of ds_read_b128, so the dim-major layout halves
//      the LDS time of the V operands.
// For bf16 pages no staging registers and no LDS stores are needed.  Waves 0-3 copy K, waves
// 4-7 copy V.
//
// Software pipeline.  Per page (64 keys) and wave (32 query rows), in the transposed domain so
// that each lane owns whole query rows:
//   QK   S^T[key][row] = K . Q^T     v_mfma_f32_32x32x16_bf16, A = K from LDS, B = Q^T in VGPRs
//   SM   causal cut (only on units that reach past the wave's first row), weights exp2 of the
//        scores (already in log2 units and relative to the row's reference, see below), P^T
//        rounded to bf16; a row's 32 scores of a unit live in lanes l and l^32
//   PV   O^T[dv][row] += V^T . P^T   A = V^T from LDS (see V above), B = P^T
// The pipeline works on units of 32 keys (half a page): unit u runs SM of unit u together with
// QK of unit u+1 and PV of unit u-1.  The three are independent, so each wave's softmax VALU
// work issues in the shadow of its own MFMAs instead of waiting for them.  Iteration i of the
// page loop is units 2i+1 and 2i+2: it reads K of page i+1 and V of page i only.  Copies run
// two iterations ahead (iteration i issues K of page i+4 and V of page i+3 and its barrier
// waits for the copies of iteration i-2), so K and V each live in a ring of four LDS tiles.
// The loop is unrolled over four iterations so that every ring tile is named statically; the
// compiler can then tell the tiles being read from the ones being filled and never waits for a
// copy early.  A wave with nothing to copy (table end) or whose page cannot be copied directly
// (an unresolved page id, or the sequence's partial last page, both written through registers
// instead) sends its copy instructions to a scratch LDS tile, so every wave issues the same
// number of copies per iteration.
//
// Softmax.  Q is taken multiplied by scale * log2(e) (rounded to bf16), so the MFMA returns
// scores in log2 units, and the first QK MFMA of a unit starts its accumulator at -m, the row's
// reference, so a weight is a bare exp2.  The reference is the row maximum of the first unit and
// is not checked against every unit's maximum: a unit whose weights in some lane sum to 2^30 or
// more (or to inf / NaN) takes a rare branch that moves the reference to the unit's row maximum,
// rescales the output accumulators (after PV of the previous unit has added the weights taken
// against the old reference) and takes the weights again.  The row sum adds the bf16-rounded
// weights that enter the PV product (v_dot2_f32_bf16 with ones, two weights per instruction), so
// the result is normalised by exactly the weights used.  This file is compiled without NaN
// semantics so that maxima need no operand quieting; NaN inputs still propagate through the
// exponentials and the MFMAs to the output.
//
// Split-KV (SPLIT): a workgroup runs one of n_splits near-equal ranges of its tile's pages and
// writes that range's normalised output (fp32) and LSE into the caller's workspace;
// split_merge_kernel combines the ranges of each row by their LSEs.
//
// Fused block union (FU): no table is given.  Each workgroup first ORs the masks of its KV
// group (the G heads over the chunk's query blocks, causally clipped) into an LDS bitmap with
// the table-build kernel's own routines (union_byte_rows, or union_bit_rows for bit-packed
// masks), and counts the set bits before each
// 64-bit word.  Table position p is the p-th set bit in ascending order, so the page ids are
// expanded from the bitmap a window chunk at a time, and the pages visited and their order are
// exactly those of the separate table-build launch: the output is bitwise the same.  Every tile
// (and with SPLIT every range of a tile) repeats the union (its masks are read from L2 after the
// first), which costs a few microseconds per workgroup against a separate launch.
#include "prefill_common.h"
#include "union_common.h"

#include <type_traits>

namespace cpa {
namespace {

constexpr int THREADS = 512;
constexpr int WIN = 1024;  // circular window of resolved page ids
constexpr int CH = 512;    // ids resolved at a time
static_assert((WIN & (WIN - 1)) == 0 && (CH & (CH - 1)) == 0 && CH <= WIN, "window sizes");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;

template <int D>
struct Geo {
  static constexpr int CPR = D / 8;     // 16-byte chunks per token row
  static constexpr int PAGE = 64 * D;   // bf16 elements of one K (or V) page
  static constexpr int NPW = CPR / 4;   // direct-to-LDS instructions per wave per page and tensor
  static constexpr int DT = D / 32;     // 32-wide output column tiles
  static constexpr int KS = D / 16;     // k-steps of the QK product
};

// chunk position of V chunk c of row r is c ^ swz_v(r)
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// fp8 token-major V staging: 16-code chunk c of token t sits at position c ^ swz_f8(t) of its
// row, so that the 8 rows of a transposed read fall in 8 different 16-byte bank groups
template <int D>
__device__ __forceinline__ int swz_f8(int t) { return D == 128 ? (t & 7) : ((t >> 2) & 1); }

// 16-byte direct-to-LDS copy: each lane's chunk at byte offset `off` from the wave-uniform
// `base` lands at ldst + 16 * lane (a 32-bit offset keeps the base in scalar registers)
__device__ __forceinline__ void lds_dma16(const char* base, uint32_t off, __bf16* ldst) {
  const char* g = base + off;
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)ldst, 16, 0, 0);
}

__device__ __forceinline__ v4i16 ds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) char*)(__attribute__((address_space(3))) void*)p));
}

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8); }

// Workgroup barrier that waits only for this wave's LDS traffic and for all but its newest `VM`
// vector-memory operations (the copies issued in the current iteration stay in flight).  The
// asm statement keeps the compiler from moving memory accesses across it.
template <int VM>
__device__ __forceinline__ void barrier_keep_vm() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 0));
  asm volatile("s_barrier" ::: "memory");
}

template <int I>
using IC = std::integral_constant<int, I>;

// VT: the V pool is dim-major ([d][token] per page and group, row stride a.v_row_stride).
// F8: the pools hold OCP e4m3 codes.  A page is copied into an LDS staging tile as codes, 16 per
// 16-byte slot, and once the codes have landed the whole workgroup converts the page to bf16
// exactly (every e4m3 value is a bf16 value) into the operand-order tiles of the bf16 dim-major
// case; from then on the page is read as in that case, whatever the pool's V layout.
//   K, and V of a dim-major pool: staging slot 32s + m holds the codes that become slots m and
//   m + 32 of slab s of the bf16 tile (K: 16 dims of one key, V: 16 keys of one dim row); a
//   thread converts one slot per tensor and page.
//   V of a token-major pool: staging holds natural rows of 16-code chunks (chunk c of token t at
//   position c ^ swz_f8(t), so that the reads below avoid bank conflicts).  ds_read_b64_tr_b8
//   transposes bytes within 16 lanes: lane s supplies half s % 2 of a 16-byte row s / 2, and
//   lane j receives byte j of each of the 8 rows.  With the rows at 8 consecutive tokens of one
//   16-dim chunk, lane j gets 8 consecutive keys of dim j: one bf16 operand slot after conversion.
// Converting once per workgroup instead of once per reading wave costs 1/8 of the conversions.
// The pipeline runs one page further ahead: iteration i copies K codes of page i+5 and V codes
// of page i+4, converts K of page i+2 and V of page i+1 (copied in iteration i-3), and reads K
// of page i+1 and V of page i, so the staging rings hold four pages and the bf16 rings two.
// The K scale is folded into the softmax scale and the V scale into the output (a.out_scale).
template <int D, bool SPLIT, bool VT, bool F8, bool FU>
__global__ __launch_bounds__(THREADS) void prefill_bf16_kernel(const PrefillArgs a) {
  using GE = Geo<D>;
  constexpr bool VOP = VT || F8;   // V tiles in operand order (8 keys of one dim per slot)
  constexpr int NPW = F8 ? (GE::NPW / 2 > 0 ? GE::NPW / 2 : 1) : GE::NPW;   // copies per wave and page
  constexpr int EB = F8 ? 1 : 2;                                            // bytes per pool element
  __shared__ __attribute__((aligned(1024))) __bf16 kR0[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 kR1[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 kR2[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 kR3[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 vR0[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 vR1[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 vR2[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 vR3[GE::PAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sink[NPW * 512];  // target of idle copies
  __shared__ int win_kb[WIN];
  __shared__ int win_ph[WIN];
  // FU: the group's block bitmap and, per word, the set bits before it
  __shared__ unsigned long long uw[FU ? MAX_KV_WORDS : 1];
  __shared__ int upre[FU ? MAX_KV_WORDS : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;  // lane half

  int gi, rank, split;
  if (!decode_tile<FU>(a, lane, gi, rank, split)) return;
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

  int cnt;
  const int32_t* tab = nullptr;
  int nwords = 0;
  if constexpr (FU) {
    // the union over the group's rows, clamped as the table-build kernel clamps its lengths
    // (prefix_blocks = qb0, chunk_blocks = nqb)
    const int uqb0 = min(qb0, a.mask_nkvb);
    const int unqb = min(min(nqb, a.mask_nqb), a.mask_nkvb - uqb0);
    nwords = (uqb0 + unqb + 63) >> 6;
    for (int w = tid; w < nwords; w += THREADS) uw[w] = 0ull;
    __syncthreads();
    uint4* red = reinterpret_cast<uint4*>(kR0);   // scratch until the first page copies
    const size_t grow = ((size_t)b * a.Hq + (size_t)g * a.G) * a.mask_nqb;   // the group's first row
    if (a.mask_bits != nullptr) {
      union_bit_rows<THREADS, 8>(a.mask_bits + grow * a.mask_words, (size_t)a.mask_words, a.mask_nqb, a.G, uqb0, unqb,
                                 uw, reinterpret_cast<unsigned long long*>(red));
    } else {
      const uint8_t* gbase = a.masks + grow * a.mask_nkvb;
      if (a.mask_vec)
        union_byte_rows<THREADS, 8, true>(gbase, (size_t)a.mask_nkvb, a.mask_nqb, a.G, uqb0, unqb, a.mask_nkvb, uw,
                                          red);
      else
        union_byte_rows<THREADS, 8, false>(gbase, (size_t)a.mask_nkvb, a.mask_nqb, a.G, uqb0, unqb, a.mask_nkvb, uw,
                                           red);
    }
    // exclusive prefix of the set bits over words: within waves by shuffles, then over the
    // wave totals
    constexpr int WPT = MAX_KV_WORDS / THREADS;
    int pc[WPT];
    int mine = 0;
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int w = tid * WPT + k;
      pc[k] = w < nwords ? __popcll(uw[w]) : 0;
      mine += pc[k];
    }
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int* tsum = reinterpret_cast<int*>(red);
    if (lane == 63) tsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int x = 0; x < THREADS / 64; ++x) {
      const int t = tsum[x];
      before += x < wave ? t : 0;
      total += t;
    }
    int run = before + incl - mine;
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int w = tid * WPT + k;
      if (w < nwords) upre[w] = run;
      run += pc[k];
    }
    __syncthreads();
    cnt = total;
  } else {
    cnt = min(max(a.counts[gi], 0), a.table_cap);
    tab = a.tables + (size_t)gi * a.table_cap;
  }
  // FU: set bits of the bitmap past block lim (the table entries with id > lim); wave-uniform
  auto bits_above = [&](int lim) __attribute__((always_inline)) {
    const int first = lim + 1;
    int c = 0;
    for (int w0 = first >> 6; w0 < nwords; w0 += 64) {
      const int w = w0 + lane;
      unsigned long long x = w < nwords ? uw[w] : 0ull;
      if (w == (first >> 6)) x &= ~0ull << (first & 63);
      c += __popcll(x);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
    // every lane holds the total: say so, so that the loop bounds derived from it stay scalar
    return __builtin_amdgcn_readfirstlane(c);
  };
  int n_iter, n_vis;
  if constexpr (FU) {
    n_iter = cnt - bits_above(qb0 + qi_last);
    n_vis = active ? cnt - bits_above(qb0 + qi_w) : 0;
  } else {
    n_iter = cnt - count_above(tab, cnt, nqb, qb0 + qi_last, lane);
    n_vis = active ? cnt - count_above(tab, cnt, nqb, qb0 + qi_w, lane) : 0;
  }
  int toff = 0;   // FU: table position of this range's first page
  if (SPLIT) {   // this workgroup's range: the tile's pages cut into n_splits near-equal ranges
    const int len = (n_iter + a.n_splits - 1) / a.n_splits;
    const int lo = min(n_iter, split * len);
    const int hi = min(n_iter, lo + len);
    if constexpr (FU) toff = lo;
    else tab += lo;
    n_vis = max(0, min(n_vis, hi) - lo);
    n_iter = max(0, hi - lo);
  }

  const char* __restrict__ kg = reinterpret_cast<const char*>(a.k) + (size_t)g * a.head_stride * EB;
  const char* __restrict__ vg = reinterpret_cast<const char*>(a.v) + (size_t)g * a.v_head_stride * EB;
  const int32_t* __restrict__ pmap = a.page_map + (size_t)b * a.page_map_stride;

  // ---- Q in registers (B operand of S^T = K Q^T) -------------------------------------------
  const int row0 = 64 * qi_w + 32 * half;   // first chunk row of this wave
  const int row = row0 + l32;               // this lane's chunk row
  const bool row_ok = active && row < Cn;
  const __bf16* qsrc = reinterpret_cast<const __bf16*>(a.q) + ((size_t)(q0 + (row_ok ? row : 0)) * a.Hq + head) * D;
  // Q is taken pre-multiplied by the softmax scale and log2(e) (rounded back to bf16), so that
  // the scores come out of the MFMA in log2 units
  const float cs = a.scale_log2;
  bf16x8 qb[GE::KS];
#pragma unroll
  for (int ks = 0; ks < GE::KS; ++ks) {
    const uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qsrc + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);
    const bf16x8 raw = __builtin_bit_cast(bf16x8, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[ks][e] = (__bf16)((float)raw[e] * cs);
  }

  // ---- direct-to-LDS plan ------------------------------------------------------------------
  // waves 0-3 move K, waves 4-7 move V; wave w's instruction j fills the 1 KiB slab
  // s = NPW w' + j of its tensor's tile (w' = w % 4), lane l the 16-byte slot l of that slab.
  const bool vrole = wave >= 4;
  const char* const tg = vrole ? vg : kg;  // this wave's tensor of group g
  const int64_t pstride = (vrole ? a.v_page_stride : a.page_stride) * EB;   // bytes
  const int rs = (int)(vrole ? a.v_row_stride : a.token_stride);   // elements between rows
  uint32_t dma_off[NPW];   // byte offset of the lane's source chunk within a page
  int dma_row[NPW];        // its (first) token
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const int sl = (wave & 3) * NPW + j;
    if (F8) {   // staging slot 64 sl + l: slots l % 32 and l % 32 + 32 of bf16 slab sb = 2 sl + l / 32
      const int sb = 2 * sl + hl;
      if (vrole && !VT) {   // natural rows: staging slot p holds chunk p % C8 ^ swz_f8(t) of token t = p / C8
        constexpr int C8 = D / 16;
        const int p = 64 * sl + lane;
        const int t = p / C8;
        dma_row[j] = t;
        dma_off[j] = (uint32_t)(t * rs + 16 * ((p % C8) ^ swz_f8<D>(t)));
      } else if (vrole) {   // slab ((2h + u) DT + dt): dim row 32dt + l % 32, keys 32h + 16u .. +15
        const int tok = 16 * (sb / GE::DT), dt = sb % GE::DT;
        dma_row[j] = tok;
        dma_off[j] = (uint32_t)((32 * dt + l32) * rs + tok);
      } else {       // slab (h, ks): key 32h + key_perm(l % 32), dims 16ks .. +15
        const int r = 32 * (sb / GE::KS) + key_perm(l32), ks = sb % GE::KS;
        dma_row[j] = r;
        dma_off[j] = (uint32_t)(r * rs + 16 * ks);
      }
    } else if (vrole && VT) {   // operand order: slab (h, u, dt), 8 keys of column 32dt + l % 32
      const int h = sl / (2 * GE::DT), u = (sl / GE::DT) & 1, dt = sl % GE::DT;
      const int tok = 32 * h + 16 * u + 8 * hl;
      dma_row[j] = tok;
      dma_off[j] = (uint32_t)((32 * dt + l32) * rs + tok) * 2u;
    } else {
      int r, c;
      if (vrole) {   // natural rows, swizzled chunks
        const int p = sl * 64 + lane;
        r = p / GE::CPR;
        c = (p % GE::CPR) ^ swz_v<D>(r);
      } else {       // operand order: slab (h, ks)
        r = 32 * (sl / GE::KS) + (VT ? key_perm(l32) : l32);
        c = 2 * (sl % GE::KS) + hl;
      }
      dma_row[j] = r;
      dma_off[j] = (uint32_t)(r * rs + c * 8) * 2u;
    }
  }
  const int dma_dst = (wave & 3) * NPW * 64 * 8;  // elements; + j * 512

  // A copy is planned at the top of an iteration and issued one direct-to-LDS instruction at a
  // time in between the iteration's MFMAs.  Pages that are unresolved (NaN) or end inside the
  // sequence (rows past the end read as 0) are written through registers at once; their copy
  // instructions, like those of an idle wave, read page 0 of the pool into the sink tile.
  struct Fill {
    const char* src;   // this wave's tensor (K or V) of the page
    __bf16* dst;       // this wave's part of the destination tile
  };
  const Fill idle{tg, sink};
  auto plan = [&](bool valid, int kb, int ph, __bf16* tile) __attribute__((always_inline)) {
    if (!valid) return idle;
    const int nv_tok = min(max(L - 64 * kb, 0), 64);
    if (ph >= 0 && nv_tok == 64) return Fill{tg + (size_t)ph * pstride, tile + dma_dst};
    const char* src = tg + (size_t)(ph < 0 ? 0 : ph) * pstride;
    const uint32_t fv = ph < 0 ? (F8 ? 0x7F7F7F7Fu : 0x7FC07FC0u) : 0u;
    constexpr int KPC = 16 / EB;   // keys in a dim-major chunk
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      uint4 v = make_uint4(fv, fv, fv, fv);
      if (ph >= 0 && dma_row[j] < nv_tok) {
        v = *reinterpret_cast<const uint4*>(src + dma_off[j]);
        if (vrole && VT && dma_row[j] + KPC > nv_tok) {   // a chunk of keys crossing the end
          unsigned char by[16];
          *reinterpret_cast<uint4*>(by) = v;
#pragma unroll
          for (int e = 0; e < KPC; ++e)
            if (dma_row[j] + e >= nv_tok)
#pragma unroll
              for (int y = 0; y < EB; ++y) by[e * EB + y] = 0;
          v = *reinterpret_cast<const uint4*>(by);
        }
      }
      *reinterpret_cast<uint4*>(tile + dma_dst + j * 512 + lane * 8) = v;
    }
    return idle;
  };
  auto fill_one = [&](const Fill& f, int j) __attribute__((always_inline)) {
    lds_dma16(f.src, dma_off[j], f.dst + j * 512);
  };
  auto fill_all = [&](const Fill& f) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NPW; ++j) fill_one(f, j);
  };

  // resolve table entries [base, base + CH) into window slots (base + j) mod WIN (indices are
  // non-negative and WIN, CH powers of two)
  auto resolve = [&](int pos, int kb) __attribute__((always_inline)) {
    int ph = -1;
    if (kb >= 0 && kb < a.page_map_stride) {
      ph = pmap[kb];
      if (ph < 0 || (int64_t)ph >= a.n_pages) ph = -1;
    }
    win_kb[pos & (WIN - 1)] = kb;
    win_ph[pos & (WIN - 1)] = ph;
  };
  auto load_chunk = [&](int base) __attribute__((always_inline)) {
    if constexpr (FU) {
      // table position p is the p-th set bit: lane l of the wave on word w holds position
      // upre[w] + (its rank among the word's set bits) when bit l is set; the range's entry j
      // is position toff + j
      const int lo_p = toff + base, hi_p = toff + min(base + CH, n_iter);
      for (int w = wave; w < nwords; w += THREADS / 64) {
        const unsigned long long word = uw[w];
        const int p0 = upre[w];
        if (p0 >= hi_p || p0 + (int)__popcll(word) <= lo_p) continue;
        const int pos = p0 + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(word >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)word, 0u));
        if (((word >> lane) & 1ull) && pos >= lo_p && pos < hi_p) resolve(pos - toff, (w << 6) + lane);
      }
    } else {
      for (int j = tid; j < CH && base + j < n_iter; j += THREADS) resolve(base + j, tab[base + j]);
    }
  };

  // ---- per-lane LDS read offsets (elements) ---------------------------------------------------
  // K operand of k-step ks, key half h: slot `lane` of slab (h, ks)
  const int k_lane_off = lane * 8;
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
  // Scores are kept relative to the row's reference m_run (log2 units): the first MFMA of each
  // QK product starts from cm = -m_run instead of 0, so a weight is exp2 of the score as it
  // comes.  The reference is set from the first unit and moves (rarely) when a row maximum
  // exceeds it by more than 2^8; the accumulators, the row sum and the scores taken against the
  // old reference then follow.
  const bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
  float m_run = 0.f;
  float l_run = 0.f;         // this lane's share of the row sum
  f32x16 cm;
#pragma unroll
  for (int j = 0; j < 16; ++j) cm[j] = 0.f;
  f32x16 o[GE::DT];
#pragma unroll
  for (int dt = 0; dt < GE::DT; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[dt][j] = 0.f;
  const int row_pos = P + row;
  const int wave_pos0 = P + row0;

  // scores of the unit in softmax and of the unit in QK (the two alternate), and the bf16
  // weights of two units as PV operands
  f32x16 sx, sy;
  bf16x8 px0, px1, py0, py1;

  // ---- the three stages, on units of 32 keys (page half h) ----------------------------------
  // QK: S^T = K Q^T for half h of the page in LDS tile Kl; copy instructions j0 .. j0+NJ-1 of f
  // go out in between
  constexpr int NJ = NPW / 2 > 0 ? NPW / 2 : 1;   // copy instructions per unit
  // F8: converts staging slot t of a page (codes at src) into slots t % 32 and t % 32 + 32 of
  // slab t / 32 of the bf16 tile dst
  constexpr int NS = GE::PAGE / 16;   // staging slots of one tensor's page
  auto convert_slot = [&](const __bf16* src, __bf16* dst, int t) __attribute__((always_inline)) {
    const uint4 c = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(src) + 16 * t);
    __bf16* d = dst + (t >> 5) * 512 + (t & 31) * 8;
    *reinterpret_cast<uint4*>(d) = fp8x8_to_bf16(make_uint2(c.x, c.y));
    *reinterpret_cast<uint4*>(d + 256) = fp8x8_to_bf16(make_uint2(c.z, c.w));
  };
  // F8, token-major V: lane item v of a page (src, natural rows) into the bf16 tile dst.  Group
  // v / 16 is key octet m and 16-dim chunk c; lane v % 16 reads half of one of the 8 rows and
  // receives dim 16c + v % 16 of keys 8m .. 8m+7, which is slot 32(m % 2) + (16c + v % 16) % 32 of
  // slab (2(m / 4) + (m / 2) % 2) DT + (16c + v % 16) / 32.
  auto convert_tr = [&](const __bf16* src, __bf16* dst, int v) __attribute__((always_inline)) {
    constexpr int C8 = D / 16;
    const int grp = v >> 4, s16 = v & 15;
    const int m = grp & 7, c = grp >> 3;
    const int t = 8 * m + (s16 >> 1);
    const __attribute__((address_space(3))) char* lp =
        (const __attribute__((address_space(3))) char*)(const __attribute__((address_space(3))) void*)src +
        16 * (t * C8 + (c ^ swz_f8<D>(t))) + 8 * (s16 & 1);
    const v2i32 codes = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)lp);
    const int col = 16 * c + s16;
    const int slab = (2 * (m >> 2) + ((m >> 1) & 1)) * GE::DT + (col >> 5);
    __bf16* d = dst + slab * 512 + (32 * (m & 1) + (col & 31)) * 8;
    *reinterpret_cast<uint4*>(d) = fp8x8_to_bf16(make_uint2((uint32_t)codes[0], (uint32_t)codes[1]));
  };
  // F8: V lane items per page: NS staging slots (dim-major pool) or 2 NS transposed reads
  constexpr int NV8 = VT ? NS : 2 * NS;
  // F8: conversion item `it` of this thread in an iteration: item x = tid + 512 it is staging slot
  // x of the K page (x < NS) or V item x - NS (wave-uniform choice)
  auto convert_item = [&](int it, const __bf16* ksrc, __bf16* kdst, const __bf16* vsrc, __bf16* vdst)
      __attribute__((always_inline)) {
    const int x = tid + THREADS * it;
    if (VT) {
      const bool isv = x >= NS;
      if (x < 2 * NS) convert_slot(isv ? vsrc : ksrc, isv ? vdst : kdst, isv ? x - NS : x);
    } else if (x < NS) {
      convert_slot(ksrc, kdst, x);
    } else if (x < NS + NV8) {
      convert_tr(vsrc, vdst, x - NS);
    }
  };
  auto qk = [&](const __bf16* Kl, int h, f32x16& s, const f32x16& c0, const Fill& f, int j0)
      __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < GE::KS; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kl + k_lane_off + (h * GE::KS + ks) * 512);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[ks], ks == 0 ? c0 : s, 0, 0, 0);
      if (ks % (GE::KS / NJ) == 0 && j0 + ks / (GE::KS / NJ) < NPW) fill_one(f, j0 + ks / (GE::KS / NJ));
    }
  };
  // SM, causal cut of half h of page kb: key position must not exceed the row position
  auto causal = [&](f32x16& s, int kb, int h) __attribute__((always_inline)) {
    const int k0 = 64 * kb + 32 * h;
    if (k0 + 31 > wave_pos0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // accumulator row 8(j/4) + 4hl + j%4 holds that key, or its key_perm image
        const int key = k0 + (VOP ? 16 * (j >> 3) + 8 * hl + (j & 7) : 8 * (j >> 2) + 4 * hl + (j & 3));
        if (key > row_pos) s[j] = -INFINITY;
      }
    }
  };
  // SM, row maximum of a unit's scores (over the 32 keys held by lanes l and l^32)
  auto rowmax = [&](const f32x16& s) __attribute__((always_inline)) {
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int j = 3; j < 15; j += 2) mx = fmaxf(fmaxf(mx, s[j]), s[j + 1]);
    return xhalf_max(fmaxf(mx, s[15]));
  };
  // SM, move the reference of the rows in which this unit's maximum mx exceeds it by more than
  // the threshold: d = mx there, 0 elsewhere; the unit's scores, the row sum and cm follow at
  // once, the accumulators (alpha = 2^-d) once PV of the previous unit is in
  auto move_reference = [&](f32x16& s, float mx, float& d, float& alpha) __attribute__((always_inline)) {
    d = mx > kRescaleThreshold ? mx : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] -= d;
#pragma unroll
    for (int j = 0; j < 16; ++j) cm[j] -= d;
    m_run += d;
    alpha = __builtin_amdgcn_exp2f(-d);
    l_run *= alpha;
  };
  // SM, weights of scores s (left as they are) against the reference, rounded to bf16 as the PV
  // operands; returns this lane's sum of them.
  //   key of operand u (0, 1), element e, lane half hl: 16*u + 8*(e / 4) + 4*hl + e % 4, or with
  //   dim-major V (key_perm) 16*u + 8*hl + e
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
  // PV: O^T += V^T P^T for half h of the page in LDS tile Vl
  auto pv = [&](const __bf16* Vl, int h, const bf16x8& p0, const bf16x8& p1) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int krow = (32 * h + 16 * u) * D;
#pragma unroll
      for (int dt = 0; dt < GE::DT; ++dt) {
        bf16x8 va;
        if (VOP) {
          va = *reinterpret_cast<const bf16x8*>(Vl + ((2 * h + u) * GE::DT + dt) * 512 + k_lane_off);
        } else {
          const v4i16 lo = ds_read_tr(Vl + krow + v_off[dt]);
          const v4i16 hi = ds_read_tr(Vl + krow + 8 * D + v_off[dt]);
          const v4i16 both[2] = {lo, hi};
          va = __builtin_bit_cast(bf16x8, both);
        }
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, u == 0 ? p0 : p1, o[dt], 0, 0, 0);
      }
    }
  };
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < GE::DT; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;
  };
  // One unit: SM of the scores in sm (half hs of page kbs) into weights pc0/pc1, QK of half hq
  // of the page in tile Kq into sq, PV of half hv of the page in tile Vp with weights pp0/pp1.
  // Apart from the causal cut (on the last pages only) and the reference move, it is one basic
  // block, so that the scheduler can interleave the three stages.  The weights are taken against
  // the current reference without looking at the unit's maximum first: a lane whose 16 weights
  // sum to kSumLimit or more (a weight of 2^26 or more), or to inf or NaN, sends the wave down the
  // rare branch, which moves the reference to the row maximum and takes the weights again.
  auto unit = [&](f32x16& sm, int kbs, int hs, bf16x8& pc0, bf16x8& pc1, const __bf16* Kq, int hq, f32x16& sq,
                  const __bf16* Vp, int hv, const bf16x8& pp0, const bf16x8& pp1,
                  const Fill& f, int j0) __attribute__((always_inline)) {
    causal(sm, kbs, hs);
    __builtin_amdgcn_s_setprio(1);
    qk(Kq, hq, sq, cm, f, j0);
    __builtin_amdgcn_s_setprio(0);
    float lu = weights(sm, pc0, pc1);
    pv(Vp, hv, pp0, pp1);
    // the weights belong to this block: keep the compiler from sinking their computation past
    // the branch below into the next unit
    asm volatile("" ::"v"(pc0), "v"(pc1), "v"(lu));
    if (__builtin_amdgcn_ballot_w64(!(lu < kSumLimit))) {
      float d, alpha;
      move_reference(sm, rowmax(sm), d, alpha);
      lu = weights(sm, pc0, pc1);
      rescale(alpha);                            // PV of the previous unit is in
#pragma unroll
      for (int j = 0; j < 16; ++j) sq[j] -= d;   // taken against the old reference
    }
    l_run += lu;
  };

  // ---- page loop ---------------------------------------------------------------------------
  // A wave computes the pages [0, n_vis) of the table; the workgroup walks [0, n_iter), and
  // n_iter > n_vis only for waves on earlier query blocks of a multi-block tile.  Per wave:
  //   prologue     QK of units 0 and 1, SM of unit 0
  //   i in [0, n_vis - 1)    iteration i in full (units 2i+1, 2i+2)
  //   i = n_vis - 1          drain: SM of unit 2i+1, PV of units 2i and 2i+1
  //   i in [n_vis, n_iter)   copies and barriers only
  if (n_iter > 0) {
    load_chunk(0);
    __syncthreads();
    auto kb_at = [&](int j) __attribute__((always_inline)) { return win_kb[j & (WIN - 1)]; };
    auto ph_at = [&](int j) __attribute__((always_inline)) { return win_ph[j & (WIN - 1)]; };
    auto kr = [&](int t) __attribute__((always_inline)) { return t == 0 ? kR0 : t == 1 ? kR1 : t == 2 ? kR2 : kR3; };
    auto vr = [&](int t) __attribute__((always_inline)) { return t == 0 ? vR0 : t == 1 ? vR1 : t == 2 ? vR2 : vR3; };
    // F8: bf16 pages in tiles 0 and 1, the four staging pages of codes in tiles 2 and 3
    auto kst = [&](int s) __attribute__((always_inline)) { return (s < 2 ? kR2 : kR3) + (s & 1) * (GE::PAGE / 2); };
    auto vst = [&](int s) __attribute__((always_inline)) { return (s < 2 ? vR2 : vR3) + (s & 1) * (GE::PAGE / 2); };
    // tiles of iteration i, r = i mod 4: K read by QK (page i+1), V read by PV (page i), and the
    // destination of this wave's copy (K of page i + fo, V of page i + fo, below)
    auto k_tile = [&](int r) __attribute__((always_inline)) { return F8 ? kr((r + 1) & 1) : kr((r + 1) & 3); };
    auto v_tile = [&](int r) __attribute__((always_inline)) { return F8 ? vr(r & 1) : vr(r & 3); };
    auto copy_tile = [&](int r) __attribute__((always_inline)) {
      if (F8) return vrole ? vst(r & 3) : kst((r + 1) & 3);
      return vrole ? vr((r + 3) & 3) : kr(r & 3);
    };
    // F8, iteration i: item `it` of the conversion of K page i+2 (staging (i+2) mod 4 -> bf16
    // (i+2) mod 2) and V page i+1 (staging (i+1) mod 4 -> bf16 (i+1) mod 2).  Pages past the
    // table convert stale codes into tiles nobody reads.
    constexpr int NIT = F8 ? (NS + NV8 + THREADS - 1) / THREADS : 0;   // items per thread and iteration
    auto convert_all = [&](int r) __attribute__((always_inline)) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) convert_item(it, kst((r + 2) & 3), kr(r & 1), vst((r + 1) & 3), vr((r + 1) & 1));
    };
    Fill fm1;
    if (F8) {
      // prologue: codes of K pages 0-2 and V pages 0-1 (iterations -5 .. -3 of the copy schedule)
      // land; those of K page 3 and V page 2 go out; K pages 0, 1 and V page 0 are converted;
      // the copies of K page 4 and V page 3 go out during the prologue's QK
      if (!vrole) {
        fill_all(plan(true, kb_at(0), ph_at(0), kst(0)));
        fill_all(plan(n_iter > 1, kb_at(1), ph_at(1), kst(1)));
        fill_all(plan(n_iter > 2, kb_at(2), ph_at(2), kst(2)));
      } else {
        fill_all(plan(true, kb_at(0), ph_at(0), vst(0)));
        fill_all(plan(n_iter > 1, kb_at(1), ph_at(1), vst(1)));
      }
      barrier_keep_vm<0>();
      fill_all(vrole ? plan(n_iter > 2, kb_at(2), ph_at(2), vst(2)) : plan(n_iter > 3, kb_at(3), ph_at(3), kst(3)));
      for (int t = tid; t < NS; t += THREADS) {
        convert_slot(kst(0), kR0, t);
        convert_slot(kst(1), kR1, t);
      }
      for (int v = tid; v < NV8; v += THREADS) {
        if (VT) convert_slot(vst(0), vR0, v);
        else convert_tr(vst(0), vR0, v);
      }
      barrier_keep_vm<NPW>();
      fm1 = vrole ? plan(n_iter > 3, kb_at(3), ph_at(3), vst(3)) : plan(n_iter > 4, kb_at(4), ph_at(4), kst(0));
    } else {
      // prologue copies: K of pages 0, 1 and V of page 0 resident; K of pages 2, 3 and V of pages
      // 1, 2 in flight (the copies of iterations -2 and -1)
      if (!vrole) {
        fill_all(plan(true, kb_at(0), ph_at(0), kR0));
        fill_all(plan(n_iter > 1, kb_at(1), ph_at(1), kR1));
      } else {
        fill_all(plan(true, kb_at(0), ph_at(0), vR0));
      }
      barrier_keep_vm<0>();
      fill_all(vrole ? plan(n_iter > 1, kb_at(1), ph_at(1), vR1) : plan(n_iter > 2, kb_at(2), ph_at(2), kR2));
      fm1 = vrole ? plan(n_iter > 2, kb_at(2), ph_at(2), vR2) : plan(n_iter > 3, kb_at(3), ph_at(3), kR3);
    }
    if (n_vis > 0) {
      qk(kR0, 0, sx, cm, fm1, 0);   // cm = 0: raw scores
      causal(sx, kb_at(0), 0);
      // the first reference: the row maximum of unit 0 (a key of it is visible to every row)
      const float mx = rowmax(sx);
      m_run = mx > -INFINITY ? mx : 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        sx[j] -= m_run;
        cm[j] = -m_run;
      }
      qk(kR0, 1, sy, cm, fm1, NJ);
      l_run = weights(sx, px0, px1);
    } else {
      fill_all(fm1);
    }
    asm volatile("s_barrier" ::: "memory");

    // Ids used by iteration i: pages i and i+1 (causal cut) and page i + fo, the one this wave
    // copies.  Those of iteration i+2 are read from the window during iteration i and held in
    // registers, so the reads' latency is covered by the iteration's work.  Slots past the table
    // hold stale ids; they are read but never used (every use is guarded by the page's range).
    constexpr int FOK = F8 ? 5 : 4;   // iteration i copies K of page i + FOK, V of page i + FOK - 1
    const int fo = vrole ? FOK - 1 : FOK;
    int vzero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
    int kb_c0 = kb_at(0), kb_c1 = kb_at(1), kb_c1n = kb_at(2);
    int kb_f = kb_at(fo), ph_f = ph_at(fo), kb_fn = kb_at(fo + 1), ph_fn = ph_at(fo + 1);
    // end of iteration i: resolve the next chunk of the window when entry i + 2 + FOK (the
    // furthest read below) starts one, read the ids of iteration i+2, shift the queue
    auto advance = [&](const int i) __attribute__((always_inline)) {
      if (((i + 2 + FOK) & (CH - 1)) == 0 && i + 2 + FOK < n_iter) {
        load_chunk(i + 2 + FOK);
        __syncthreads();
      }
      // the fresh ids stay in vector registers (the opaque zero in the slot index keeps the
      // compiler from moving them to scalar registers, which would wait for the reads here);
      // they move to scalar registers one iteration later, long after the reads completed
      const int l_kb = kb_at(i + 3 + vzero), l_kbf = kb_at(i + 2 + fo + vzero), l_phf = ph_at(i + 2 + fo + vzero);
      kb_c0 = kb_c1;
      kb_c1 = __builtin_amdgcn_readfirstlane(kb_c1n);
      kb_c1n = l_kb;
      kb_f = __builtin_amdgcn_readfirstlane(kb_fn);
      ph_f = __builtin_amdgcn_readfirstlane(ph_fn);
      kb_fn = l_kbf;
      ph_fn = l_phf;
    };
    // iteration i (R = i mod 4): units 2i+1 and 2i+2 on K of page i+1 and V of page i; this
    // wave's copy of page i + fo; with F8 the conversions of the iteration, last, where a wave
    // would otherwise wait at the barrier for the others (measured faster than placing them
    // before or between the units, or inside the units' blocks)
    auto step = [&](auto Rc, const int i) __attribute__((always_inline)) {
      constexpr int r = decltype(Rc)::value;
      const Fill f = plan(i + fo < n_iter, kb_f, ph_f, copy_tile(r));
      unit(sy, kb_c0, 1, py0, py1, k_tile(r), 0, sx, v_tile(r), 0, px0, px1, f, 0);
      unit(sx, kb_c1, 0, px0, px1, k_tile(r), 1, sy, v_tile(r), 1, py0, py1, f, NJ);
      convert_all(r);
      barrier_keep_vm<2 * NPW>();
      advance(i);
    };
    // copies (and conversions) and barrier only (the wave has no page i)
    auto idle_step = [&](const int i) __attribute__((always_inline)) {
      const int r = i & 3;
      fill_all(plan(i + fo < n_iter, kb_f, ph_f, copy_tile(r)));
      convert_all(r);
      barrier_keep_vm<2 * NPW>();
      advance(i);
    };

    const int n_full = n_vis - 1;   // iterations in full
    int i = 0;
    for (; i + 4 <= n_full; i += 4) {
      step(IC<0>{}, i);
      step(IC<1>{}, i + 1);
      step(IC<2>{}, i + 2);
      step(IC<3>{}, i + 3);
    }
    if (i < n_full) {
      step(IC<0>{}, i);
      if (i + 1 < n_full) step(IC<1>{}, i + 1);
      if (i + 2 < n_full) step(IC<2>{}, i + 2);
      i = n_full;
    }
    if (n_vis > 0) {
      // drain (iteration n_vis - 1): SM of its last unit, PV of its last two units
      const int r = i & 3;
      fill_all(plan(i + fo < n_iter, kb_f, ph_f, copy_tile(r)));
      convert_all(r);
      causal(sy, kb_c0, 1);
      float lu = weights(sy, py0, py1);
      const bool moved = __builtin_amdgcn_ballot_w64(!(lu < kSumLimit)) != 0;
      float d = 0.f, alpha = 1.f;
      if (moved) {
        move_reference(sy, rowmax(sy), d, alpha);
        lu = weights(sy, py0, py1);
      }
      l_run += lu;
      pv(v_tile(r), 0, px0, px1);
      if (moved) rescale(alpha);
      pv(v_tile(r), 1, py0, py1);
      barrier_keep_vm<2 * NPW>();
      advance(i);
      ++i;
    }
    for (; i < n_iter; ++i) idle_step(i);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));  // idle copies into the sink have landed
  }

  // ---- epilogue ----------------------------------------------------------------------------
  if (!row_ok) return;
  const float lt = xhalf_sum(l_run);
  const float inv = lt > 0.f ? a.out_scale / lt : 0.f;   // out_scale: the fp8 V scale, else 1
  if (SPLIT) {   // normalised partial output and LSE of this range, fp32
    if (q0 + row >= a.total_q) return;   // rows past total_q (inconsistent cu_q) have no slot
    const size_t rh = (size_t)split * a.total_q * a.Hq + (size_t)(q0 + row) * a.Hq + head;
    float* pdst = a.part_o + rh * D;
#pragma unroll
    for (int dt = 0; dt < GE::DT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = make_float4(o[dt][4 * q] * inv, o[dt][4 * q + 1] * inv, o[dt][4 * q + 2] * inv,
                                     o[dt][4 * q + 3] * inv);
        *reinterpret_cast<float4*>(pdst + 32 * dt + 8 * q + 4 * hl) = v;
      }
    if (hl == 0) a.part_lse[rh] = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
    return;
  }
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

// Split-KV merge: one wave per (row, head) combines the n_splits normalised partials by their
// LSEs, O = sum_s e^(lse_s - LSE) O_s with LSE = log sum_s e^lse_s (empty ranges have
// lse = -inf and weigh nothing), and writes the bf16 output and the LSE.
template <int D>
__global__ __launch_bounds__(256) void split_merge_kernel(const MergeArgs m) {
  constexpr int PL = D / 64;   // values per lane
  const size_t rh = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t n_rh = (size_t)m.total_q * m.Hq;
  if (rh >= n_rh) return;
  const int lane = threadIdx.x & 63;
  float mx = -INFINITY;
  for (int s = 0; s < m.n_splits; ++s) mx = fmaxf(mx, m.part_lse[s * n_rh + rh]);
  float acc[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) acc[e] = 0.f;
  float sum = 0.f;
  if (mx > -INFINITY) {
    for (int s = 0; s < m.n_splits; ++s) {
      const float w = __builtin_amdgcn_exp2f((m.part_lse[s * n_rh + rh] - mx) * 1.4426950408889634f);
      sum += w;
      const float* src = m.part_o + (s * n_rh + rh) * D + lane * PL;
#pragma unroll
      for (int e = 0; e < PL; ++e) acc[e] += w * src[e];
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  __bf16* dst = reinterpret_cast<__bf16*>(m.o) + rh * D + lane * PL;
#pragma unroll
  for (int e = 0; e < PL; ++e) dst[e] = (__bf16)(acc[e] * inv);
  if (m.lse != nullptr && lane == 0) m.lse[rh] = sum > 0.f ? mx + __logf(sum) : -INFINITY;
}

template <int D>
hipError_t launch_bf16(const PrefillArgs& a, hipStream_t s) {
  const int grid = prefill_grid(a);
  if (grid == 0) return hipSuccess;
  const bool split = a.n_splits > 1;
  const dim3 g(grid), t(THREADS);
  if (a.fused && a.kv_fp8) {   // fp8 pages
    if (a.v_dmajor) {
      if (split) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, true, true>), g, t, 0, s, a);
      else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, true, true, true>), g, t, 0, s, a);
    } else {
      if (split) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, true, true>), g, t, 0, s, a);
      else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, true, true>), g, t, 0, s, a);
    }
    return hipGetLastError();
  }
  if (a.fused) {   // bf16 pages
    if (a.v_dmajor) {
      if (split) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, false, true>), g, t, 0, s, a);
      else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, true, false, true>), g, t, 0, s, a);
    } else {
      if (split) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, false, true>), g, t, 0, s, a);
      else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, false, true>), g, t, 0, s, a);
    }
    return hipGetLastError();
  }
  if (a.kv_fp8) {   // fp8 pages
    if (a.v_dmajor) {
      if (split) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, true, false>), g, t, 0, s, a);
      else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, true, true, false>), g, t, 0, s, a);
    } else {
      if (split) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, true, false>), g, t, 0, s, a);
      else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, true, false>), g, t, 0, s, a);
    }
    return hipGetLastError();
  }
  if (a.v_dmajor) {
    if (split) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, false, false>), g, t, 0, s, a);
    else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, true, false, false>), g, t, 0, s, a);
  } else {
    if (split) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, false, false>), g, t, 0, s, a);
    else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, false, false>), g, t, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_merge(const MergeArgs& m, int d, hipStream_t s) {
  const size_t n_rh = (size_t)m.total_q * m.Hq;
  if (n_rh == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_rh + 3) / 4));
  if (d == 64) hipLaunchKernelGGL((split_merge_kernel<64>), grid, dim3(256), 0, s, m);
  else hipLaunchKernelGGL((split_merge_kernel<128>), grid, dim3(256), 0, s, m);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int d, hipStream_t s) {
  if (a.fused)   // the caller has checked: bf16 q, row strides within 32-bit offsets
    return d == 64 ? launch_bf16<64>(a, s) : launch_bf16<128>(a, s);
  if (a.kv_fp8 && (a.token_stride > (1 << 24) || a.v_row_stride > (1 << 24)))
    return launch_prefill_regstaged(a, true, d, s);   // fp8 strides past the direct-to-LDS kernel's offsets
  if (!bf16) return launch_prefill_regstaged(a, false, d, s);
  if (a.token_stride > (1 << 24) || a.v_row_stride > (1 << 24))   // 32-bit offsets within a page
    return launch_prefill_regstaged(a, true, d, s);
  return d == 64 ? launch_bf16<64>(a, s) : launch_bf16<128>(a, s);
}

}  // namespace cpa
