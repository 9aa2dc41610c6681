"""cpa_chunked_prefill_split_static (the split-KV call with its partials in the library's own
per-device array, for callers that cannot allocate) against cpa_chunked_prefill_split with a
caller workspace: the same kernels on the same inputs, so the outputs must be bitwise equal.
Two calls in a row, the second with a smaller input, so that the second reads partials over a
region the first left filled."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_reduce_amd as cpa
from workloads import make_workload
from workloads.configs import mask_bernoulli

from _gpu import compare, gpu_tables, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def bern(p, local=1):
    return lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=local)


CASES = [  # (name, prefix lengths, chunk lengths, Hq, Hkv, d, split_pages): larger first
    ("big", [8192, 2048], [1024, 300], 8, 2, 128, 32),
    ("small", [1024], [256], 8, 2, 64, 8),
]


def test_static_scratch_matches_workspace_split():
    for name, P, C, Hq, Hkv, d, sp in CASES:
        print(f"\n[case] split static scratch {name} split_pages={sp}", flush=True)
        w = make_workload(name, P, C, Hq, Hkv, d, "bf16", bern(0.2), 41)
        dv = upload(w)
        tables, counts = gpu_tables(dv, w)
        need = cpa.split_workspace_bytes(w.q.shape[0], Hq, d, w.nkvb_max, sp)
        assert 0 < need <= cpa.api.STATIC_SCRATCH_BYTES
        o1, l1 = cpa.chunked_prefill(dv["q"], dv["kp"], dv["vp"], dv["pm"], tables, counts, dv["cu"], dv["pl"],
                                     w.max_chunk_len, return_lse=True, split_pages=sp)
        o2 = torch.empty_like(o1)
        l2 = torch.empty_like(l1)
        r2 = cpa.chunked_prefill_split_static(dv["q"], dv["kp"], dv["vp"], dv["pm"], tables, counts, dv["cu"],
                                              dv["pl"], w.max_chunk_len, sp, out=o2, lse=l2)
        torch.cuda.synchronize()
        assert r2[0] is o2 and r2[1] is l2
        assert torch.equal(o1, o2), f"{name}: outputs differ"
        assert torch.equal(l1, l2), f"{name}: LSE differ"
        T, Cn = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
        O, _ = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, Cn, w.cu_q, w.prefix_len, w.Hkv)
        compare(w, o2, O, f"static scratch {name}")


def test_static_scratch_refuses_more_than_its_size():
    # 64 MiB holds ceil(cap / split) * Tq * Hq * (d + 1) floats: this call needs twice that
    w = make_workload("cap", [1024], [256], 8, 2, 64, "bf16", bern(0.2), 42)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    big_q = torch.zeros((8192, 128, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cpa.CpaError) as e:
        cpa.chunked_prefill_split_static(big_q, dv["kp"], dv["vp"], dv["pm"], tables, counts, dv["cu"], dv["pl"],
                                         w.max_chunk_len, 4)
    assert e.value.status == 5
