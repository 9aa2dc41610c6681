"""KV append written out: each chunk row of new K and V goes to its slot of the paged cache.

"CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract: the
chunk attends over KV blocks read in place from a paged cache, so its own K/V rows are in that
cache before attention runs (the reading that the chunk's K/V are appended first).  Row r of
sequence b is token position p = prefix_len[b] + r; it lives in logical block p // 64, whose
physical page is page_map[b][p // 64], at slot p % 64.  A logical block past the page map's
width, or a page id outside [0, n_pages), has no page: such rows are not written.

Test infrastructure, like the rest of this package.
"""
import numpy as np

BLOCK = 64


def append_kv(k_new, v_new, k_pages, v_pages, page_map, cu_q, prefix_len):
    """Copies of the pools [n_pages][Hkv][64][d] with every chunk row written to its slot.

    k_new, v_new: [Tq][Hkv][d]; rows of sequence b at cu_q[b]..cu_q[b+1].  One row at a time,
    in the order of the definition above.
    """
    k_out = np.array(k_pages, copy=True)
    v_out = np.array(v_pages, copy=True)
    n_pages = k_out.shape[0]
    for b in range(len(prefix_len)):
        for r in range(int(cu_q[b + 1] - cu_q[b])):
            p = int(prefix_len[b]) + r
            blk = p // BLOCK
            if blk >= page_map.shape[1]:
                continue
            page = int(page_map[b, blk])
            if page < 0 or page >= n_pages:
                continue
            k_out[page, :, p % BLOCK, :] = k_new[cu_q[b] + r]
            v_out[page, :, p % BLOCK, :] = v_new[cu_q[b] + r]
    return k_out, v_out
