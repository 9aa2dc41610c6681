"""Block-Union KV Selection for chunked prefill on MI355X (gfx950).

Thin wrappers over the C ABI in include/cpa.h:

* build_block_tables(masks, prefix_blocks, chunk_blocks, Hkv) -> (tables, counts)
* build_block_tables_bits(mask_bits, nkvb_max, prefix_blocks, chunk_blocks, Hkv): the same from
  bit-packed masks (one bit per block)
* chunked_prefill(q, k_pages, v_pages, page_map, tables, counts, cu_q, prefix_len,
                  max_chunk_len, split_pages=0, v_layout="token") -> (o, lse)
  (split_pages > 0: split-KV over page ranges with an LSE merge; plan_split_pages picks one,
  split_pages="auto" applies it for the device;
  v_layout "dim": V pages stored [page][group][d][64])
* build_block_plans(masks, prefix_blocks, chunk_blocks) and chunked_prefill_direct(...): the
  direct block-sparse baseline, every (head, query block) over its own mask row
* chunked_prefill_fused(q, k_pages, v_pages, page_map, masks, cu_q, prefix_len, max_chunk_len,
                        v_layout="token") -> (o, lse): the table build and the prefill in one
  launch (each workgroup builds its group's union from the masks)
* append_kv(k_new, v_new, k_pages, v_pages, page_map, cu_q, prefix_len, max_chunk_len,
            v_layout="token"): the chunk's K/V rows into the paged cache

The library must be built first (``python -m sparse_attention_long_reduce_amd.build``); nothing
here falls back to another implementation.
"""
from .api import (  # noqa: F401
    BLOCK,
    append_kv,
    attention_flops,
    build_block_plans,
    build_block_tables,
    build_block_tables_bits,
    chunked_prefill,
    chunked_prefill_direct,
    chunked_prefill_fused,
    chunked_prefill_split_static,
    plan_flops,
    plan_split_pages,
    prefill_tiles,
    split_workspace_bytes,
    status_string,
    version,
)
from ._lib import CpaError, EXPORTS, LIB_PATH, load  # noqa: F401
