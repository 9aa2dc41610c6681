"""Direct block-sparse attention: every (head, query block) over its own mask row, in float64
(test infrastructure; see package header).

Source: "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection",
abstract: the point of comparison of the block-union tables is block-sparse execution that runs
each head's mask as it is.  Definition computed:
  * the plan of (b, h, qi) is the blocks kb with masks[b][h][qi][kb] != 0 and kb <= qb0 + qi
    (qb0 = prefix_len[b] / 64), ascending; rows qi >= chunk_blocks[b] have none;
  * row r of query block qi = r // 64 attends over the tokens t of its plan's blocks with
    t <= prefix_len[b] + r, of KV group h // (Hq / Hkv), with the exact two-pass softmax of
    paged_attention (same scale, same empty-row convention).
"""
import math

import numpy as np

from .attention import _gather_group, _softmax_rows

BLOCK = 64


def block_plans(masks, prefix_blocks, chunk_blocks, plan_cap):
    """masks [B][Hq][nqb_max][nkvb_max] -> (plans int32 [B][Hq][nqb_max][plan_cap], counts)."""
    masks = np.asarray(masks)
    B, Hq, nqb_max, nkvb_max = masks.shape
    if plan_cap < nkvb_max:
        raise ValueError("plan_cap must be >= nkvb_max")
    plans = np.full((B, Hq, nqb_max, plan_cap), -1, dtype=np.int32)
    counts = np.zeros((B, Hq, nqb_max), dtype=np.int32)
    for b in range(B):
        qb0, nqb = int(prefix_blocks[b]), int(chunk_blocks[b])
        for qi in range(min(nqb, nqb_max)):
            lim = min(qb0 + qi + 1, nkvb_max)
            for h in range(Hq):
                ids = np.nonzero(masks[b, h, qi, :lim])[0]
                plans[b, h, qi, :ids.size] = ids
                counts[b, h, qi] = ids.size
    return plans, counts


def _rows_of_block(q, k_pages, v_pages, page_map, plans, counts, cu_q, prefix_len, Hkv, b, h, qi, rows, scale):
    G = q.shape[1] // Hkv
    g = h // G
    blocks = plans[b, h, qi, :counts[b, h, qi]]
    K, V, pos = _gather_group(k_pages, v_pages, page_map[b], blocks, g)
    Q = q[cu_q[b] + rows, h, :].astype(np.float64)
    S = (Q @ K.T) * scale
    p = int(prefix_len[b]) + rows
    return _softmax_rows(S, pos[None, :] <= p[:, None], V)


def block_sparse_attention(q, k_pages, v_pages, page_map, plans, counts, cu_q, prefix_len, Hkv, scale=None):
    """All rows.  -> O float64 [Tq][Hq][d], LSE float64 [Hq][Tq]."""
    Tq, Hq, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    O = np.zeros((Tq, Hq, d), dtype=np.float64)
    LSE = np.full((Hq, Tq), -np.inf, dtype=np.float64)
    for b in range(len(prefix_len)):
        C = int(cu_q[b + 1] - cu_q[b])
        for qi in range((C + BLOCK - 1) // BLOCK):
            rows = np.arange(BLOCK * qi, min(C, BLOCK * qi + BLOCK))
            for h in range(Hq):
                o, lse, _ = _rows_of_block(q, k_pages, v_pages, page_map, plans, counts, cu_q, prefix_len, Hkv,
                                           b, h, qi, rows, scale)
                O[cu_q[b] + rows, h] = o
                LSE[h, cu_q[b] + rows] = lse
    return O, LSE


def block_sparse_rows(q, k_pages, v_pages, page_map, plans, counts, cu_q, prefix_len, Hkv, samples, scale=None):
    """Rows given as (b, h, r) triples -> (O float64 [n][d], LSE float64 [n])."""
    d = q.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    O = np.zeros((len(samples), d))
    L = np.zeros(len(samples))
    for i, (b, h, r) in enumerate(samples):
        o, lse, _ = _rows_of_block(q, k_pages, v_pages, page_map, plans, counts, cu_q, prefix_len, Hkv,
                                   int(b), int(h), int(r) // BLOCK, np.array([int(r)]), scale)
        O[i], L[i] = o[0], lse[0]
    return O, L
