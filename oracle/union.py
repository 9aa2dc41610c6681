"""Block-Union KV Selection tables, by explicit OR (test infrastructure; see package header).

Source: "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection",
abstract.  The 2D block-sparse masks (query block x KV block, per query head) are read as
KV-selection signals and turned into GQA-aware per-group KV block tables by a Q-block union
(OR over the chunk's query blocks) and an intra-group union (OR over the query heads that share
one KV head).  The result is the minimal table that still keeps every selected KV block.

Readings where the pages are silent:
  * query head h belongs to KV group h // (Hq // Hkv) (contiguous GQA grouping);
  * a mask entry (qi, kb) only counts if kb <= prefix_blocks + qi, i.e. the KV block is
    causally reachable from that query block; other entries (and padding) are ignored;
  * tables hold logical KV-block ids in ascending order, padded with -1 up to the capacity.
"""
import numpy as np


def block_union_tables(masks, prefix_blocks, chunk_blocks, Hkv, table_cap):
    """masks uint8 [B][Hq][nqb_max][nkvb_max] (nonzero = selected) -> (tables, counts).

    tables int32 [B][Hkv][table_cap]; counts int32 [B][Hkv].
    """
    masks = np.asarray(masks)
    B, Hq, nqb_max, nkvb_max = masks.shape
    G = Hq // Hkv
    tables = np.full((B, Hkv, table_cap), -1, dtype=np.int32)
    counts = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        qb0 = int(prefix_blocks[b])
        nqb = int(chunk_blocks[b])
        nkvb = qb0 + nqb
        qi = np.arange(nqb)[:, None]
        kb = np.arange(nkvb)[None, :]
        reachable = kb <= qb0 + qi                      # [nqb][nkvb]
        sel = (masks[b, :, :nqb, :nkvb] != 0) & reachable[None]   # [Hq][nqb][nkvb]
        for g in range(Hkv):
            heads = sel[g * G:(g + 1) * G]              # the query heads of group g
            union = heads.any(axis=(0, 1))              # OR over heads and Q-blocks
            ids = np.nonzero(union)[0].astype(np.int32)  # ascending
            if ids.size > table_cap:
                raise ValueError("table capacity too small")
            tables[b, g, :ids.size] = ids
            counts[b, g] = ids.size
    return tables, counts


def unpack_mask_bits(mask_bits, nkvb_max):
    """Bit-packed masks uint64 [B][Hq][nqb][words] -> bool [B][Hq][nqb][nkvb_max]: block kb is
    selected iff bit kb % 64 of word kb // 64 is set (the packed input format)."""
    bits = np.asarray(mask_bits, dtype=np.uint64)
    kb = np.arange(nkvb_max)
    words = bits[..., kb // 64]
    return ((words >> (kb % 64).astype(np.uint64)) & np.uint64(1)).astype(bool)


def block_union_tables_bits(mask_bits, nkvb_max, prefix_blocks, chunk_blocks, Hkv, table_cap=None):
    """The tables of the bit-packed masks: those of the masks they encode."""
    return block_union_tables(unpack_mask_bits(mask_bits, nkvb_max).astype(np.uint8), prefix_blocks,
                              chunk_blocks, Hkv, nkvb_max if table_cap is None else table_cap)
