// Device code of the block union (Q-block union and intra-group union) shared by the table-build
// kernel and the fused prefill.
//
// "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract: the
// masks of the chunk's query blocks and of the query heads that share one KV head are ORed into
// one per-group set of KV blocks.
#pragma once
#include "cpa_internal.h"

namespace cpa {

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

// OR of the byte-mask rows of one (sequence, KV group) into a bitmap, called by all NT threads
// of a workgroup.  Row (head hh < G of the group, query block qi < nqb) starts at
// gbase + (hh * nqb_rows + qi) * row_stride and holds one byte per KV block (row_stride >=
// nkvb_max bytes, nonzero = selected).  On return bit kb of words[] is set iff some row has a
// nonzero byte at kb <= qb0 + qi (the causal clip: block kb is reachable from query block qi),
// for kb < qb0 + nqb.  words[] holds ceil((qb0 + nqb) / 64) words and must be zero on entry;
// red is NT x 16 bytes of LDS scratch.  Ends with a barrier.
//
// The columns of 16 blocks (one 16-byte load per row, VEC; else byte loads bounded by
// nkvb_max) are spread over the threads, each column's rows over NT / cols threads that walk
// them by stepping (no division per row) with RIF loads in flight.  The partial ORs of one
// column meet in red by a tree; the bytes are ORed before they become bits, and the clip only
// touches rows whose causal limit falls inside the column.
template <int NT, int RIF, bool VEC>
__device__ __forceinline__ void union_byte_rows(const uint8_t* gbase, size_t row_stride, int nqb_rows, int G,
                                                int qb0, int nqb, int nkvb_max, unsigned long long* words,
                                                uint4* red) {
  const int tid = threadIdx.x;
  const int nchunk = (qb0 + nqb + 15) >> 4;
  int lg = 0;
  while ((1 << lg) < nchunk && (1 << lg) < NT) ++lg;
  const int cols = 1 << lg;
  const int rsplit = NT >> lg;

  for (int c0 = 0; c0 < nchunk; c0 += cols) {
    const int c = c0 + (tid & (cols - 1));
    const int s = tid >> lg;
    uint32_t acc[4] = {0u, 0u, 0u, 0u};
    const int kb0 = c << 4;
    const int qi_lo = max(0, kb0 - qb0);  // first query block that can reach column kb0
    const int nq = nqb - qi_lo;
    if (c < nchunk && nq > 0) {
      // mask bytes of row (head hh of the group, query block qi) at column kb0, causally clipped
      auto row = [&](int hh, int qi, uint32_t v[4]) __attribute__((always_inline)) {
        const uint8_t* rowp = gbase + ((size_t)hh * nqb_rows + qi) * row_stride + kb0;
        if (VEC) {
          const uint4 x = *reinterpret_cast<const uint4*>(rowp);
          v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else {
          const int lim = min(16, nkvb_max - kb0);
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
      // row t = (head hh, query block qi_lo + qr), walked from t = s in steps of rsplit rows
      // without a division per row
      int hh = s / nq, qr = s - (s / nq) * nq;
      const int dh = rsplit / nq, dq = rsplit - (rsplit / nq) * nq;
      for (int t0 = s; t0 < nrows; t0 += RIF * rsplit) {
        uint32_t v[RIF][4];
#pragma unroll
        for (int u = 0; u < RIF; ++u) {
          if (t0 + u * rsplit < nrows) {
            row(hh, qi_lo + qr, v[u]);
          } else {
            v[u][0] = v[u][1] = v[u][2] = v[u][3] = 0u;
          }
          qr += dq;
          hh += dh;
          if (qr >= nq) {
            qr -= nq;
            ++hh;
          }
        }
#pragma unroll
        for (int u = 0; u < RIF; ++u)
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
}

// OR of the bit-packed mask rows of one (sequence, KV group) into a bitmap, called by all NT
// threads of a workgroup: the same union and causal clip as union_byte_rows, for rows of
// mask_words 64-bit words (bit kb % 64 of word kb / 64 = block kb selected).  Row (head hh,
// query block qi) starts at wbase + (hh * nqb_rows + qi) * wstride.  words[] holds
// ceil((qb0 + nqb) / 64) words and must be zero on entry; redw is NT x 8 bytes of LDS scratch.
// Ends with a barrier.  A thread ORs whole words of its column over its rows (RIF loads in
// flight), the clip is a word mask, and the row splits of a column meet by a tree.
template <int NT, int RIF>
__device__ __forceinline__ void union_bit_rows(const unsigned long long* wbase, size_t wstride, int nqb_rows,
                                               int G, int qb0, int nqb, unsigned long long* words,
                                               unsigned long long* redw) {
  const int tid = threadIdx.x;
  const int nwords = (qb0 + nqb + 63) >> 6;
  int lgw = 0;
  while ((1 << lgw) < nwords && (1 << lgw) < NT) ++lgw;
  const int colw = 1 << lgw;
  const int rs = NT >> lgw;
  for (int c0 = 0; c0 < nwords; c0 += colw) {
    const int c = c0 + (tid & (colw - 1));
    const int s = tid >> lgw;
    unsigned long long acc = 0ull;
    const int kb0 = c << 6;
    const int qi_lo = max(0, kb0 - qb0);
    const int nq = nqb - qi_lo;
    if (c < nwords && nq > 0) {
      const int nrows = G * nq;
      // row t = (head hh, query block qi_lo + qr), walked from t = s in steps of rs rows
      // without a division per row
      int hh = s / nq, qr = s - (s / nq) * nq;
      const int dh = rs / nq, dq = rs - (rs / nq) * nq;
      for (int t0 = s; t0 < nrows; t0 += RIF * rs) {
        unsigned long long v[RIF];
#pragma unroll
        for (int u = 0; u < RIF; ++u) {
          v[u] = 0ull;
          if (t0 + u * rs < nrows) {
            const int qi = qi_lo + qr;
            v[u] = wbase[((size_t)hh * nqb_rows + qi) * wstride + c];
            const int nallow = qb0 + qi - kb0 + 1;   // bits 0 .. nallow-1 are causally reachable (>= 1)
            if (nallow < 64) v[u] &= (1ull << nallow) - 1ull;
          }
          qr += dq;
          hh += dh;
          if (qr >= nq) {
            qr -= nq;
            ++hh;
          }
        }
#pragma unroll
        for (int u = 0; u < RIF; ++u) acc |= v[u];
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

}  // namespace cpa
