/*
 * cpa.h - C ABI of the Block-Union KV Selection hot path for chunked prefill (MI355X, gfx950).
 *
 * The method is CompactAttention's Block-Union KV Selection ("CompactAttention: Accelerating
 * Chunked Prefill with Block-Union KV Selection", abstract): per-head 2D block-sparse masks over
 * (query block, KV block) are treated as KV-selection signals, not as kernel execution plans.
 * A union over the chunk's query blocks and a union over the query heads that share one KV head
 * turn them into the minimal per-group KV block tables that keep every selected block; attention
 * for every query head of the group then reads exactly those blocks in place from the paged KV
 * cache, with no KV compaction.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise.  The caller allocates
 *     and owns every buffer; the library allocates no device memory and keeps no global state,
 *     so concurrent calls on different streams are safe.  The one exception is
 *     cpa_chunked_prefill_split_static, whose partials live in a device array of the library
 *     (see there).
 *   - Calls only enqueue work on `stream` (0 = the default stream) and return without
 *     synchronising.  Results are visible in stream order.
 *   - Block size: query blocks, KV blocks and KV pages all hold CPA_BLOCK = 64 tokens.
 *   - GQA grouping: query head h belongs to KV group h / (Hq / Hkv).
 *   - Size limits (CPA_ERR_SHAPE beyond them): strides at most 2^40 elements, at most 65536
 *     query heads, B * Hkv at most INT_MAX, and at most INT_MAX workgroups per launch (KV
 *     groups x query tiles x split ranges for the prefill; sequences x chunk pages x KV groups
 *     for the append).  Far beyond any pool that fits in memory, they keep every size product
 *     the checks and the kernels form from overflowing.
 *   - Host-side argument checks run before any HIP call; on failure nothing is enqueued and a
 *     CPA_ERR_* code is returned.  Device-resident data (lengths, tables, page ids) cannot be
 *     checked on the host: the kernels clamp every index they derive from it so that no access
 *     leaves the buffers described here, and the per-call notes say what such data must satisfy
 *     for the result to be meaningful.  The exception is the row offsets cu_q, which address q,
 *     o and the new K/V rows, buffers whose extent the library is not told: cu_q must be
 *     non-decreasing with cu_q[B] equal to the buffers' row count Tq.
 */
#ifndef CPA_H
#define CPA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CPA_BLOCK 64
#define CPA_MAX_KV_BLOCKS 65536 /* per sequence: 4M tokens */

typedef enum {
  CPA_OK = 0,
  CPA_ERR_NULL = 1,        /* a required pointer is NULL                                   */
  CPA_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, or inconsistent */
  CPA_ERR_ALIGN = 3,       /* a pointer or stride breaks the alignment stated below         */
  CPA_ERR_UNSUPPORTED = 4, /* dtype, head dim or path the library does not implement      */
  CPA_ERR_CAPACITY = 5,    /* table capacity smaller than the KV-block count               */
  CPA_ERR_LAUNCH = 6       /* the HIP runtime rejected a kernel launch                      */
} cpa_status;

typedef enum {
  CPA_F32 = 0,
  CPA_BF16 = 1,
  CPA_FP8_E4M3 = 2 /* OCP e4m3 (bias 7, no infinities); KV pools only (cpa_chunked_prefill_fp8kv,
                      cpa_chunked_prefill_fused(_bits), cpa_append_kv) */
} cpa_dtype;

/*
 * cpa_build_block_tables - masks -> minimal GQA-aware per-group KV block tables + counts.
 *
 * Implements the Q-block union and the intra-group union of the CompactAttention abstract:
 * logical KV block kb is in the table of (sequence b, KV group g) iff some query head h of
 * group g and some query block qi of b's chunk have masks[b][h][qi][kb] != 0 with
 * kb <= prefix_blocks[b] + qi (the block is causally reachable from that query block).
 * Entries outside that causal region, and padding past a sequence's extent, are ignored.
 *
 *   masks          uint8 [B][Hq][nqb_max][nkvb_max], nonzero = selected.
 *   prefix_blocks  int32 [B]: prefix length of sequence b in blocks (first query block's
 *                  absolute block index).
 *   chunk_blocks   int32 [B]: query blocks in sequence b's chunk (ceil(chunk_len / 64)).
 *                  Device values are clamped to [0, nqb_max] and prefix + chunk to nkvb_max.
 *   tables   (out) int32 [B][Hkv][table_cap]: selected logical KV-block ids in strictly
 *                  ascending order, then -1 up to table_cap.  Requires table_cap >= nkvb_max.
 *   counts   (out) int32 [B][Hkv]: number of ids in each table.
 *
 * Errors: CPA_ERR_NULL (any pointer NULL with B > 0), CPA_ERR_SHAPE (B, Hq, Hkv, nqb_max,
 * nkvb_max negative; Hkv == 0; Hq % Hkv != 0; nkvb_max > CPA_MAX_KV_BLOCKS),
 * CPA_ERR_CAPACITY (table_cap < nkvb_max), CPA_ERR_LAUNCH.
 * The result is bit-exact: it has exactly one correct value.
 */
cpa_status cpa_build_block_tables(const uint8_t* masks, int B, int Hq, int Hkv, int nqb_max,
                                  int nkvb_max, const int32_t* prefix_blocks,
                                  const int32_t* chunk_blocks, int32_t* tables, int table_cap,
                                  int32_t* counts, hipStream_t stream);

/*
 * cpa_build_block_tables_bits - cpa_build_block_tables for bit-packed masks: one bit per
 * (query head, query block, KV block) instead of one byte, so the mask read is 8x smaller.
 * The tables and counts are those cpa_build_block_tables returns for the unpacked masks (the
 * same Q-block and intra-group union of the CompactAttention abstract, same causal clip).
 *
 *   mask_bits   uint64 [B][Hq][nqb_max][mask_words]: block kb of row (b, h, qi) is selected iff
 *               bit kb % 64 of word kb / 64 is set.  8-byte aligned.
 *   mask_words  64-bit words per row, >= ceil(nkvb_max / 64); bits at or past nkvb_max and
 *               outside the causal region are ignored.
 * Other arguments and errors as cpa_build_block_tables, plus CPA_ERR_SHAPE for
 * mask_words < ceil(nkvb_max / 64) and CPA_ERR_ALIGN for a misaligned mask_bits.
 */
cpa_status cpa_build_block_tables_bits(const uint64_t* mask_bits, int B, int Hq, int Hkv, int nqb_max,
                                       int nkvb_max, int mask_words, const int32_t* prefix_blocks,
                                       const int32_t* chunk_blocks, int32_t* tables, int table_cap,
                                       int32_t* counts, hipStream_t stream);

/*
 * cpa_chunked_prefill - attention of one prefill chunk per sequence over the selected blocks.
 *
 * For every sequence b, query head h (group g = h / (Hq/Hkv)) and chunk row r (absolute
 * position p = prefix_len[b] + r), attends over the key tokens t of the blocks
 * tables[b][g][0 .. counts[b][g]) with t <= p (causal cut on the chunk's own blocks), reading
 * K/V in place from the paged cache through page_map; fp32 online softmax with scale sm_scale.
 * This is the step of the CompactAttention abstract that reads the selected KV blocks where
 * they lie in the cache, without first gathering them into a compact copy.
 *
 *   q        [Tq][Hq][d] in `dtype`, d contiguous; rows of sequence b are cu_q[b] .. cu_q[b+1]
 *            (Tq = cu_q[B]).  16-byte aligned.
 *   k_pages, v_pages  paged cache in `dtype`: element (page, kv head, token-in-page, c) at
 *            page*page_stride + head*head_stride + token*token_stride + c (strides in elements,
 *            c contiguous); the dense layout [n_pages][Hkv][64][d] has page_stride = Hkv*64*d,
 *            head_stride = 64*d, token_stride = d.  Base pointers 16-byte aligned and every
 *            stride a multiple of 16 bytes.
 *   n_pages  physical pages in the pool, >= 1 when there is work (B > 0, max_chunk_len > 0;
 *            else CPA_ERR_SHAPE).  A page id outside [0, n_pages), or a table entry outside
 *            [0, page_map_stride), is never dereferenced: its keys and values read as NaN.
 *   page_map int32 [B][page_map_stride]: logical KV block -> physical page.
 *   tables, counts, table_cap  as produced by cpa_build_block_tables (ids ascending; counts are
 *            clamped to table_cap).
 *   cu_q     int32 [B+1], prefix_len int32 [B]: device arrays; cu_q non-decreasing from 0 to
 *            Tq; prefix_len[b] must be a multiple of 64 (it is the absolute position of the
 *            chunk's first row) and the chunk's own K/V must already be in the cache.  Chunk
 *            lengths are clamped to max_chunk_len.
 *   max_chunk_len  host int >= every chunk length (sizes the grid).
 *   sm_scale softmax scale, > 0; pass 0 for 1/sqrt(d).
 *   o  (out) [Tq][Hq][d] in `dtype`.  A row with no visible key gets zeros.
 *   lse (out, optional) float [Tq][Hq]: natural-log sum-exp of the scaled scores (-inf for a
 *            row with no visible key).  NULL to skip.
 *
 * Supported: dtype CPA_BF16 (bf16 MFMA, fp32 accumulation and softmax, P rounded to bf16
 * before the PV product) and CPA_F32 (fp32 MFMA end to end); d in {64, 128};
 * G = Hq/Hkv any divisor (a workgroup takes four (query block, head) pairs of one group).
 * Errors: CPA_ERR_NULL, CPA_ERR_SHAPE (negative sizes, Hq % Hkv != 0, table_cap < 0,
 * page_map_stride < 1 or n_pages < 1 with work to do, strides too small to hold a page),
 * CPA_ERR_ALIGN, CPA_ERR_UNSUPPORTED (dtype, d), CPA_ERR_LAUNCH.
 */
cpa_status cpa_chunked_prefill(const void* q, cpa_dtype dtype, const void* k_pages,
                               const void* v_pages, int64_t page_stride, int64_t head_stride,
                               int64_t token_stride, int64_t n_pages, const int32_t* page_map,
                               int page_map_stride, const int32_t* tables, int table_cap,
                               const int32_t* counts, const int32_t* cu_q,
                               const int32_t* prefix_len, int B, int Hq, int Hkv, int d,
                               int max_chunk_len, float sm_scale, void* o, float* lse,
                               hipStream_t stream);

/*
 * cpa_chunked_prefill_split - cpa_chunked_prefill with the pages each (group, query tile)
 * visits cut into n_splits near-equal ranges (split-KV), for calls with too few tiles to fill
 * the GPU or with tables of very different lengths.
 *
 * Each range is run by its own workgroup, which writes the normalised partial output of its
 * rows and their LSE over that range into `workspace`.  A second kernel then combines the
 * ranges of each row, O = sum_s e^(lse_s - LSE) O_s with LSE = log sum_s e^lse_s, and writes
 * o and lse.  The result equals cpa_chunked_prefill's up to rounding (the partials are fp32).
 * Softmax over the union of a partition of the keys is the LSE-weighted merge of the softmaxes
 * over the parts; the CompactAttention abstract's per-group tables are unchanged.
 *
 * Arguments as cpa_chunked_prefill, plus:
 *   total_q     rows of all sequences (Tq = cu_q[B]); sizes the workspace rows.
 *   split_pages >= 1; sets n_splits = ceil(table_cap / split_pages) ranges per tile.  A tile
 *               that visits n pages gives each range ceil(n / n_splits) of them (the last ones
 *               fewer), at most split_pages.  With n_splits == 1 this is cpa_chunked_prefill and
 *               the workspace is unused.
 *   workspace   device memory owned by the caller, 16-byte aligned, at least
 *               cpa_split_workspace_bytes(total_q, Hq, d, table_cap, split_pages) bytes; its
 *               contents on entry do not matter and on return are unspecified.  Calls that use
 *               the same workspace must not overlap.
 * Supported: dtype CPA_BF16 with token_stride <= 2^24 elements (else CPA_ERR_UNSUPPORTED
 * when n_splits > 1).  Errors: those of cpa_chunked_prefill, CPA_ERR_SHAPE (split_pages < 1,
 * total_q < 0), CPA_ERR_NULL (no workspace), CPA_ERR_ALIGN, CPA_ERR_CAPACITY (workspace too
 * small).
 */
cpa_status cpa_chunked_prefill_split(const void* q, cpa_dtype dtype, const void* k_pages,
                                     const void* v_pages, int64_t page_stride, int64_t head_stride,
                                     int64_t token_stride, int64_t n_pages, const int32_t* page_map,
                                     int page_map_stride, const int32_t* tables, int table_cap,
                                     const int32_t* counts, const int32_t* cu_q,
                                     const int32_t* prefix_len, int B, int Hq, int Hkv, int d,
                                     int max_chunk_len, float sm_scale, void* o, float* lse,
                                     int total_q, int split_pages, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/*
 * cpa_chunked_prefill_split_static - cpa_chunked_prefill_split with no workspace argument and no
 * allocation of any kind, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The split partials live in a
 * device array inside the library, CPA_STATIC_SCRATCH_BYTES (64 MiB) large, that every GPU the
 * library runs on holds from the first call on that GPU until the process ends; its address on
 * a device is looked up on that first call (the stream's device, or the current one for the
 * default stream).  Same attention, kernels and results as cpa_chunked_prefill_split.
 *
 * Arguments as cpa_chunked_prefill_split without workspace / workspace_bytes.  The caller still
 * passes q, the pools, tables and the outputs.
 * Errors: those of cpa_chunked_prefill_split; CPA_ERR_CAPACITY when
 * cpa_split_workspace_bytes(total_q, Hq, d, table_cap, split_pages) exceeds
 * CPA_STATIC_SCRATCH_BYTES (checked before any HIP call); CPA_ERR_LAUNCH when the array's
 * device address cannot be obtained.  Every call on one GPU shares that GPU's array and it keeps
 * the last call's contents (nothing in it needs to start at zero: every partial the merge reads
 * is written first by the same call), so calls that overlap in time on one GPU (different
 * streams, or threads) race and must be serialised by the caller.
 */
#define CPA_STATIC_SCRATCH_BYTES (64 * 1024 * 1024)
cpa_status cpa_chunked_prefill_split_static(const void* q, cpa_dtype dtype, const void* k_pages,
                                            const void* v_pages, int64_t page_stride, int64_t head_stride,
                                            int64_t token_stride, int64_t n_pages, const int32_t* page_map,
                                            int page_map_stride, const int32_t* tables, int table_cap,
                                            const int32_t* counts, const int32_t* cu_q,
                                            const int32_t* prefix_len, int B, int Hq, int Hkv, int d,
                                            int max_chunk_len, float sm_scale, void* o, float* lse,
                                            int total_q, int split_pages, hipStream_t stream);

/* Bytes of workspace cpa_chunked_prefill_split needs (0 when it needs none, or for
 * non-positive arguments): ceil(table_cap / split_pages) * total_q * Hq * (d + 1) * 4 when
 * that split count exceeds 1. */
size_t cpa_split_workspace_bytes(int total_q, int Hq, int d, int table_cap, int split_pages);

/*
 * cpa_chunked_prefill_vt - cpa_chunked_prefill (split_pages <= 0) or cpa_chunked_prefill_split
 * (split_pages >= 1) for a V pool whose pages are stored dim-major: within a page and group the
 * d rows hold 64 consecutive tokens each, the layout [n_pages][Hkv][d][64] by default.  The K
 * pool keeps the token-major layout of cpa_chunked_prefill.  The result is the same attention
 * (CompactAttention abstract: every query head of the group over exactly its table's blocks,
 * read in place from the paged cache).  It equals cpa_chunked_prefill's on the same values up
 * to rounding: the keys of each 16-key MFMA step are summed in another order.
 *
 * Why: the PV product contracts over tokens, so its V operand is 8 consecutive tokens of one
 * column.  Dim-major pages hold those in one 16-byte chunk, which the kernel stages in LDS in
 * operand order and reads at full LDS width, instead of building each operand from two
 * half-width transposed reads.  A cache writer that stores V this way pays nothing extra.
 *
 * Arguments as cpa_chunked_prefill_split, except that V is described by its own strides
 * (elements): V(page, group, token, dim) at v_pages + page * v_page_stride +
 * group * v_head_stride + dim * v_dim_stride + token.  Requires v_dim_stride >= 64,
 * v_head_stride >= d * v_dim_stride, v_page_stride >= Hkv * v_head_stride (else CPA_ERR_SHAPE),
 * all three 16-byte multiples (else CPA_ERR_ALIGN).  total_q, workspace and workspace_bytes are
 * used only when split_pages >= 1 (see cpa_chunked_prefill_split; a split also needs
 * v_dim_stride <= 2^24, else CPA_ERR_UNSUPPORTED).
 */
cpa_status cpa_chunked_prefill_vt(const void* q, cpa_dtype dtype, const void* k_pages, int64_t page_stride,
                                  int64_t head_stride, int64_t token_stride, const void* v_pages,
                                  int64_t v_page_stride, int64_t v_head_stride, int64_t v_dim_stride,
                                  int64_t n_pages, const int32_t* page_map, int page_map_stride,
                                  const int32_t* tables, int table_cap, const int32_t* counts,
                                  const int32_t* cu_q, const int32_t* prefix_len, int B, int Hq, int Hkv,
                                  int d, int max_chunk_len, float sm_scale, void* o, float* lse, int total_q,
                                  int split_pages, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * cpa_chunked_prefill_fused - cpa_build_block_tables and cpa_chunked_prefill(_vt) in one launch:
 * the block union moves into the prefill's prologue.  Each workgroup ORs the masks of its KV
 * group itself (the Q-block union and the intra-group union of the CompactAttention abstract,
 * with the causal clip of cpa_build_block_tables) into a bitmap in LDS and walks the blocks it
 * selects in ascending order.  Neither tables nor counts are read or written.  The result is
 * bitwise that of cpa_build_block_tables with prefix_blocks[b] = prefix_len[b] / 64 and
 * chunk_blocks[b] = ceil(chunk length / 64), followed by cpa_chunked_prefill (v_dim_major = 0)
 * or cpa_chunked_prefill_vt (v_dim_major = 1) on those tables with table_cap = nkvb_max (the
 * same split ranges when split_pages >= 1); with fp8 pools, followed by
 * cpa_chunked_prefill_fp8kv with the same scales.
 *
 * Why: chunked prefill repeats the table build at every chunk (CompactAttention abstract); one
 * launch instead of two removes a launch and its gap per chunk.  Every tile of a group repeats
 * the union (the group's masks are read once from HBM, then from L2).
 *
 *   masks, nqb_max, nkvb_max  as cpa_build_block_tables (uint8 [B][Hq][nqb_max][nkvb_max],
 *            nonzero = selected; nkvb_max <= CPA_MAX_KV_BLOCKS).  Query blocks at or past
 *            nqb_max, and blocks at or past nkvb_max, select nothing (the table build's clamps).
 *            Rows are read 16 bytes at a time when nkvb_max % 16 == 0 and masks is 16-byte
 *            aligned, else a byte at a time.
 *   v_dim_major, v_page_stride, v_head_stride, v_row_stride  the V pool as cpa_append_kv
 *            describes it: token-major (0, v_row_stride = token stride) or dim-major (1,
 *            v_row_stride = dim stride).
 *   kv_dtype, k_scale, v_scale  the pools' element type: CPA_BF16 (the scales are not used), or
 *            CPA_FP8_E4M3 with the per-tensor dequantization scales of
 *            cpa_chunked_prefill_fp8kv (finite, > 0, else CPA_ERR_SHAPE; pool strides in bytes,
 *            16-byte multiples).  Any other kv_dtype: CPA_ERR_UNSUPPORTED.
 *   total_q, split_pages, workspace, workspace_bytes  split-KV as cpa_chunked_prefill_split, with
 *            nkvb_max in the place of table_cap: n_splits = ceil(nkvb_max / split_pages), and the
 *            workspace needs cpa_split_workspace_bytes(total_q, Hq, d, nkvb_max, split_pages)
 *            bytes.  split_pages <= 0: no split (total_q and the workspace are not used).  Each
 *            range's workgroup builds the union itself.
 * Other arguments as cpa_chunked_prefill.
 * Supported: dtype (of q and o) CPA_BF16, d in {64, 128}, any G, row strides (token_stride,
 * v_row_stride) up to 2^24 elements (else CPA_ERR_UNSUPPORTED).
 * Errors: those of cpa_chunked_prefill (without the table checks) and, with split_pages >= 1, of
 * cpa_chunked_prefill_split; CPA_ERR_SHAPE (v_dim_major not 0 or 1, nqb_max or nkvb_max
 * negative, nkvb_max > CPA_MAX_KV_BLOCKS), CPA_ERR_NULL (masks NULL with nqb_max, nkvb_max > 0).
 */
cpa_status cpa_chunked_prefill_fused(const void* q, cpa_dtype dtype, const void* k_pages, int64_t page_stride,
                                     int64_t head_stride, int64_t token_stride, const void* v_pages,
                                     int v_dim_major, int64_t v_page_stride, int64_t v_head_stride,
                                     int64_t v_row_stride, cpa_dtype kv_dtype, float k_scale, float v_scale,
                                     int64_t n_pages, const int32_t* page_map, int page_map_stride,
                                     const uint8_t* masks, int nqb_max, int nkvb_max,
                                     const int32_t* cu_q, const int32_t* prefix_len, int B, int Hq, int Hkv,
                                     int d, int max_chunk_len, float sm_scale, void* o, float* lse, int total_q,
                                     int split_pages, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * cpa_chunked_prefill_fused_bits - cpa_chunked_prefill_fused from bit-packed masks: the union in
 * each workgroup's prologue reads one bit per (query head, query block, KV block), 8x fewer
 * mask bytes.  The result is bitwise that of cpa_chunked_prefill_fused on the unpacked masks
 * (and of cpa_build_block_tables_bits followed by cpa_chunked_prefill(_vt)).
 *
 *   mask_bits, mask_words  as cpa_build_block_tables_bits (uint64 [B][Hq][nqb_max][mask_words],
 *            mask_words >= ceil(nkvb_max / 64), 8-byte aligned; bits at or past nkvb_max and
 *            outside the causal region are ignored).
 * Other arguments, support and errors as cpa_chunked_prefill_fused, plus CPA_ERR_SHAPE for
 * mask_words < ceil(nkvb_max / 64) and CPA_ERR_ALIGN for a misaligned mask_bits.
 */
cpa_status cpa_chunked_prefill_fused_bits(const void* q, cpa_dtype dtype, const void* k_pages, int64_t page_stride,
                                          int64_t head_stride, int64_t token_stride, const void* v_pages,
                                          int v_dim_major, int64_t v_page_stride, int64_t v_head_stride,
                                          int64_t v_row_stride, cpa_dtype kv_dtype, float k_scale, float v_scale,
                                          int64_t n_pages, const int32_t* page_map, int page_map_stride,
                                          const uint64_t* mask_bits, int nqb_max, int nkvb_max,
                                          int mask_words, const int32_t* cu_q, const int32_t* prefix_len, int B,
                                          int Hq, int Hkv, int d, int max_chunk_len, float sm_scale, void* o,
                                          float* lse, int total_q, int split_pages, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/*
 * cpa_append_kv - write each sequence's chunk of new K and V rows into the paged cache, the step
 * before attention in chunked prefill (CompactAttention abstract: the chunk attends over KV
 * blocks that live in a paged cache and are read in place, so its own K/V must be there).
 *
 *   k_new, v_new  [Tq][Hkv][d] in `dtype`, contiguous; rows of sequence b at cu_q[b]..cu_q[b+1]
 *                 (the layout of q with Hkv heads).
 *   k_pages       out: the K pool, layout as in cpa_chunked_prefill (token-major).
 *   v_pages       out: the V pool; v_dim_major = 0: token-major with (v_page_stride,
 *                 v_head_stride, v_row_stride = token stride), dim contiguous; v_dim_major = 1:
 *                 dim-major as in cpa_chunked_prefill_vt (v_row_stride = dim stride), tokens
 *                 contiguous.
 *   n_pages, page_map, page_map_stride, cu_q, prefix_len, B, Hkv, d, max_chunk_len
 *                 as in cpa_chunked_prefill.
 *
 * Row r of sequence b goes to position p = prefix_len[b] + r: slot p % 64 of physical page
 * page_map[b][p / 64], group h for head h.  Nothing else in the pools is written: slots of the
 * last page past the chunk stay as they were.  A page whose logical block is >= page_map_stride
 * or whose id is outside [0, n_pages) is skipped (its rows are not written).  A copy: the pool
 * holds the input bits exactly.  Calls must not overlap with a prefill reading the same pages.
 * Supported: CPA_BF16, CPA_F32 and CPA_FP8_E4M3 (all three tensors in that dtype), d in {64, 128}.
 * Errors: CPA_ERR_NULL, CPA_ERR_SHAPE (negative sizes, strides too small to hold a page,
 * v_dim_major not 0 or 1, page_map_stride < 1), CPA_ERR_ALIGN (16-byte alignment of pointers
 * and strides), CPA_ERR_UNSUPPORTED, CPA_ERR_LAUNCH.
 */
cpa_status cpa_append_kv(const void* k_new, const void* v_new, cpa_dtype dtype, void* k_pages,
                         int64_t page_stride, int64_t head_stride, int64_t token_stride, void* v_pages,
                         int v_dim_major, int64_t v_page_stride, int64_t v_head_stride, int64_t v_row_stride,
                         int64_t n_pages, const int32_t* page_map, int page_map_stride, const int32_t* cu_q,
                         const int32_t* prefix_len, int B, int Hkv, int d, int max_chunk_len,
                         hipStream_t stream);

/*
 * cpa_build_block_plans - per-(head, query block) KV block plans: the direct block-sparse
 * execution that the Q-block and intra-group unions of the CompactAttention abstract replace
 * (the abstract's point of comparison: running every head's mask directly pays off poorly when
 * a chunk holds only a few query blocks).  No union: row
 * (b, h, qi) of the plan lists the blocks kb with masks[b][h][qi][kb] != 0 and
 * kb <= prefix_blocks[b] + qi, ascending, then -1 up to plan_cap; rows qi >= chunk_blocks[b]
 * are empty.
 *
 *   masks, B, Hq, nqb_max, nkvb_max, prefix_blocks, chunk_blocks  as cpa_build_block_tables.
 *   plans       (out) int32 [B][Hq][nqb_max][plan_cap], plan_cap >= nkvb_max.
 *   plan_counts (out) int32 [B][Hq][nqb_max].
 * Errors: CPA_ERR_NULL, CPA_ERR_SHAPE, CPA_ERR_CAPACITY (plan_cap < nkvb_max), CPA_ERR_LAUNCH.
 * Bit-exact: the plans have exactly one correct value.
 */
cpa_status cpa_build_block_plans(const uint8_t* masks, int B, int Hq, int nqb_max, int nkvb_max,
                                 const int32_t* prefix_blocks, const int32_t* chunk_blocks, int32_t* plans,
                                 int plan_cap, int32_t* plan_counts, hipStream_t stream);

/*
 * cpa_chunked_prefill_direct - chunked-prefill attention in which every (sequence, query head,
 * query block) attends over exactly the blocks of its own plan (cpa_build_block_plans), read in
 * place from the paged cache, with the causal cut of cpa_chunked_prefill.  It is per-query
 * block-sparse attention with the original masks, the baseline the union tables are measured
 * against, on the same numerics as the bf16 path of cpa_chunked_prefill.
 *
 * Arguments as cpa_chunked_prefill_vt (token-major K, dim-major V), with the plans in place of
 * the tables: plans / plan_cap / plan_counts from cpa_build_block_plans and its nqb_max
 * (>= ceil(max_chunk_len / 64)).  o, lse as cpa_chunked_prefill: a row whose plan reaches no
 * visible key gets O = 0 and LSE = -inf; an unresolvable page id reads as NaN.
 * Supported: CPA_BF16, d in {64, 128}, G = Hq / Hkv any divisor.
 * Errors: CPA_ERR_NULL, CPA_ERR_SHAPE, CPA_ERR_ALIGN, CPA_ERR_UNSUPPORTED, CPA_ERR_LAUNCH.
 */
cpa_status cpa_chunked_prefill_direct(const void* q, cpa_dtype dtype, const void* k_pages, int64_t page_stride,
                                      int64_t head_stride, int64_t token_stride, const void* v_pages,
                                      int64_t v_page_stride, int64_t v_head_stride, int64_t v_dim_stride,
                                      int64_t n_pages, const int32_t* page_map, int page_map_stride,
                                      const int32_t* plans, int plan_cap, const int32_t* plan_counts,
                                      int nqb_max, const int32_t* cu_q, const int32_t* prefix_len, int B, int Hq,
                                      int Hkv, int d, int max_chunk_len, float sm_scale, void* o, float* lse,
                                      hipStream_t stream);

/*
 * cpa_chunked_prefill_fp8kv - cpa_chunked_prefill with bf16 q / o and a KV cache of fp8 pages
 * (OCP e4m3, one byte per element): the same attention over the same tables (CompactAttention
 * abstract), over the keys decode(k) * k_scale and values decode(v) * v_scale.  Each page is
 * copied into LDS as codes and, once they have landed, converted to bf16 once per workgroup
 * into the operand-order tiles that the bf16 dim-major path reads (token-major V is transposed
 * on the way by byte-transposing LDS reads); the conversion is exact, as bf16 holds every e4m3
 * value.  The K scale joins the softmax scale and the V scale multiplies the normalised output,
 * both in fp32.  The attention is the bf16 path's (bf16 MFMA, fp32 softmax, bf16 P).  The cache
 * takes half the memory of bf16.
 *
 *   k_pages     e4m3 pool, token-major, strides (page, head, token) in elements = bytes.
 *   v_pages     e4m3 pool, token-major (v_dim_major = 0, v_row_stride = token stride) or
 *               dim-major (v_dim_major = 1, v_row_stride = dim stride), strides in bytes.
 *   k_scale, v_scale  finite, > 0 (else CPA_ERR_SHAPE): the per-tensor dequantization scales.
 *   total_q, split_pages, workspace, workspace_bytes  split-KV as cpa_chunked_prefill_split
 *               (split_pages >= 1, pool row strides up to 2^24 bytes, else
 *               CPA_ERR_UNSUPPORTED): each range's partial output already carries v_scale, and
 *               the merge is the bf16 path's.  split_pages <= 0: no split (total_q and the
 *               workspace are not used).
 * Other arguments and errors as cpa_chunked_prefill (dtype bf16 for q and o; pool strides are
 * in bytes and must be 16-byte multiples, else CPA_ERR_ALIGN) and, with split_pages >= 1, those
 * of cpa_chunked_prefill_split.
 */
cpa_status cpa_chunked_prefill_fp8kv(const void* q, const void* k_pages, const void* v_pages, int64_t page_stride,
                                     int64_t head_stride, int64_t token_stride, int v_dim_major,
                                     int64_t v_page_stride, int64_t v_head_stride, int64_t v_row_stride,
                                     float k_scale, float v_scale, int64_t n_pages, const int32_t* page_map,
                                     int page_map_stride, const int32_t* tables, int table_cap,
                                     const int32_t* counts, const int32_t* cu_q, const int32_t* prefix_len, int B,
                                     int Hq, int Hkv, int d, int max_chunk_len, float sm_scale, void* o, float* lse,
                                     int total_q, int split_pages, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Static, NUL-terminated description of a status code (host pointer, never NULL). */
const char* cpa_status_string(cpa_status s);

/* Library version as major*10000 + minor*100 + patch. */
int cpa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CPA_H */
