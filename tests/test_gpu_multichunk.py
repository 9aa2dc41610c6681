"""GPU parity of the full chunked prefill of one 131072-token sequence run as ONE varlen launch
pair over its 64 chunks of 2048 (each chunk a sequence of the batch, prefix 2048k, all over the
same paged pool), against the oracle and against the 64 separate launches.

A tile's work does not depend on the rest of the grid, so the batched prefill must reproduce
the per-chunk launches bit for bit; the tables must match the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_reduce_amd as cpa
from workloads.configs import chunked_sequence_batch, chunked_sequence_chunk

from _gpu import compare, gpu_tables, sample_rows, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_multichunk_batch_equals_per_chunk_launches():
    print("\n[case] 64-chunk batch", flush=True)
    w = chunked_sequence_batch()
    assert w.B == 64
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    assert np.array_equal(tables.cpu().numpy(), T) and np.array_equal(counts.cpu().numpy(), C)
    vpd = dv["vp"].transpose(2, 3).contiguous()
    o, lse = cpa.chunked_prefill(dv["q"], dv["kp"], vpd, dv["pm"], tables, counts, dv["cu"], dv["pl"],
                                 w.max_chunk_len, return_lse=True, v_layout="dim")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    for k in (0, 17, 63):
        wk = chunked_sequence_chunk(k)
        dk = upload(wk, k_pages=w.k_pages, v_pages=w.v_pages)
        tk, ck = gpu_tables(dk, wk)
        ok, lk = cpa.chunked_prefill(dk["q"], dv["kp"], vpd, dk["pm"], tk, ck, dk["cu"], dk["pl"], wk.max_chunk_len,
                                     return_lse=True, v_layout="dim")
        rows = slice(int(w.cu_q[k]), int(w.cu_q[k + 1]))
        assert torch.equal(ok, o[rows]) and torch.equal(lk, lse[rows]), f"chunk {k} differs"
    S = sample_rows(w, 256, seed=7)
    S = S[np.random.default_rng(7).choice(len(S), size=min(len(S), 256), replace=False)]
    Os, Ls = oracle.attention_rows(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv, S)
    r = torch.from_numpy(w.cu_q[S[:, 0]] + S[:, 2]).cuda()
    h = torch.from_numpy(S[:, 1]).cuda()
    compare(w, o[r, h].float().cpu().numpy(), Os, "64-chunk batch")
    assert np.max(np.abs(lse[r, h].cpu().numpy() - Ls)) < 2e-2
