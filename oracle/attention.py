"""Chunked-prefill attention over the per-group KV block tables, in float64 (test infrastructure;
see package header).

Source: "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection",
abstract: every query head of a GQA group attends over exactly the KV blocks of its group's
table, which are read from the paged KV cache where they lie (the oracle may copy them; only the
device path must not).

Definition computed (readings where the pages are silent are marked R):
  * sequence b owns query rows cu_q[b] .. cu_q[b+1]; row r of its chunk sits at absolute
    position p = prefix_len[b] + r (R: the chunk's own K/V are already in the paged cache);
  * query head h uses KV group g = h // (Hq // Hkv) (R: contiguous grouping);
  * key token t of logical block kb = t // 64 is stored at k_pages[page_map[b][kb]][g][t % 64];
  * the keys of row (b, h, r) are the tokens t of the blocks in tables[b][g][:counts[b][g]]
    with t <= p (R: bottom-right causal alignment; only the chunk's own blocks are cut);
  * s_t = scale * <q, k_t> with scale = 1/sqrt(d) unless given (R);
  * exact two-pass softmax: m = max_t s_t, w_t = exp(s_t - m), O = sum_t w_t v_t / sum_t w_t,
    LSE = m + ln(sum_t w_t) (natural log);
  * a row with no key gets O = 0 and LSE = -inf (R).
"""
import math

import numpy as np

BLOCK = 64


def _gather_group(k_pages, v_pages, page_map_row, blocks, g):
    """Copy the selected blocks of KV group g into contiguous float64 arrays."""
    d = k_pages.shape[-1]
    phys = page_map_row[blocks]
    K = k_pages[phys, g].reshape(-1, d).astype(np.float64)
    V = v_pages[phys, g].reshape(-1, d).astype(np.float64)
    pos = (np.asarray(blocks, dtype=np.int64)[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    return K, V, pos


def _softmax_rows(S, visible, V):
    """S [n][m] scores, visible bool [n][m], V [m][d] -> (O [n][d], LSE [n], n_visible [n])."""
    S = np.where(visible, S, -np.inf)
    m = S.max(axis=1) if S.shape[1] else np.full(S.shape[0], -np.inf)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    w = np.exp(S - m_safe[:, None])                   # exp(-inf) = 0 for hidden keys
    l = w.sum(axis=1)
    O = np.zeros((S.shape[0], V.shape[1]), dtype=np.float64)
    O[has] = (w[has] @ V) / l[has, None]
    lse = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), -np.inf)
    return O, lse, visible.sum(axis=1)


def paged_attention(q, k_pages, v_pages, page_map, tables, counts, cu_q, prefix_len, Hkv,
                    scale=None, return_nvis=False):
    """All rows.  q float [Tq][Hq][d] -> O float64 [Tq][Hq][d], LSE float64 [Hq][Tq]."""
    Tq, Hq, d = q.shape
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    O = np.zeros((Tq, Hq, d), dtype=np.float64)
    LSE = np.full((Hq, Tq), -np.inf, dtype=np.float64)
    NV = np.zeros((Tq, Hq), dtype=np.int64)
    for b in range(len(prefix_len)):
        P = int(prefix_len[b])
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        for g in range(Hkv):
            blocks = tables[b, g, :counts[b, g]]
            K, V, pos = _gather_group(k_pages, v_pages, page_map[b], blocks, g)
            # rows are processed in batches of 64 only to bound memory; each row's result
            # depends on that row alone
            for r0 in range(0, q1 - q0, BLOCK):
                r1 = min(q1 - q0, r0 + BLOCK)
                Q = q[q0 + r0:q0 + r1, g * G:(g + 1) * G, :].astype(np.float64)   # [rows][G][d]
                rows = r1 - r0
                S = (Q.reshape(rows * G, d) @ K.T) * scale                       # [rows*G][n]
                p = P + np.arange(r0, r1)
                visible = np.repeat(pos[None, :] <= p[:, None], G, axis=0)       # row-major (row, head)
                o, lse, nv = _softmax_rows(S, visible, V)
                O[q0 + r0:q0 + r1, g * G:(g + 1) * G, :] = o.reshape(rows, G, d)
                LSE[g * G:(g + 1) * G, q0 + r0:q0 + r1] = lse.reshape(rows, G).T
                NV[q0 + r0:q0 + r1, g * G:(g + 1) * G] = nv.reshape(rows, G)
    if return_nvis:
        return O, LSE, NV
    return O, LSE


def attention_rows(q, k_pages, v_pages, page_map, tables, counts, cu_q, prefix_len, Hkv, samples,
                   scale=None, return_nvis=False):
    """Selected rows only.  samples int [n][3] of (b, h, r) with r the row within sequence b's
    chunk.  Returns O float64 [n][d] and LSE float64 [n] (and the visible-key count per row)."""
    samples = np.asarray(samples, dtype=np.int64).reshape(-1, 3)
    Tq, Hq, d = q.shape
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    O = np.zeros((len(samples), d), dtype=np.float64)
    LSE = np.full(len(samples), -np.inf, dtype=np.float64)
    NV = np.zeros(len(samples), dtype=np.int64)
    groups = {}
    for i, (b, h, r) in enumerate(samples):
        groups.setdefault((int(b), int(h) // G), []).append(i)
    for (b, g), idx in groups.items():
        blocks = tables[b, g, :counts[b, g]]
        K, V, pos = _gather_group(k_pages, v_pages, page_map[b], blocks, g)
        idx = np.asarray(idx)
        hs = samples[idx, 1]
        rs = samples[idx, 2]
        Q = q[int(cu_q[b]) + rs, hs, :].astype(np.float64)                      # [n][d]
        S = (Q @ K.T) * scale
        visible = pos[None, :] <= (int(prefix_len[b]) + rs)[:, None]
        o, lse, nv = _softmax_rows(S, visible, V)
        O[idx] = o
        LSE[idx] = lse
        NV[idx] = nv
    if return_nvis:
        return O, LSE, NV
    return O, LSE

