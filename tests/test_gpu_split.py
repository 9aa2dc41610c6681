"""GPU parity of split-KV (cpa_chunked_prefill_split) against the fp64 CPU oracle.

Splitting a tile's table into page ranges and merging the ranges by their LSEs must give the
attention over the whole table: the oracle is the same plain attention as for the unsplit path
(attention over a partition of the keys, merged by LSE, is the attention over all of them).
The bf16 tolerances are those of the unsplit path.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_reduce_amd as cpa
from workloads import make_config, make_workload
from workloads.configs import mask_all, mask_bernoulli

from _gpu import compare, gpu_tables, sample_rows, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def bern(p, local=1):
    return lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=local)


SMALL = {
    "g4_d64": dict(prefix_len=[768], chunk_len=[256], Hq=8, Hkv=2, d=64, mask_fn=bern(0.2)),
    "g2_varlen_d128": dict(prefix_len=[0, 640, 1280], chunk_len=[320, 192, 64], Hq=4, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g4_ragged_multi": dict(prefix_len=[0, 192, 4096], chunk_len=[37, 130, 255], Hq=8, Hkv=2, d=128, mask_fn=bern(0.05)),
    "g8_d128": dict(prefix_len=[512], chunk_len=[256], Hq=16, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g1_d128": dict(prefix_len=[1024, 64], chunk_len=[192, 100], Hq=2, Hkv=2, d=128, mask_fn=bern(0.3)),
    "all_zero": dict(prefix_len=[256], chunk_len=[128], Hq=8, Hkv=2, d=128, mask_fn=lambda rng, *a: mask_all(rng, *a, value=0)),
    "zero_len_chunk": dict(prefix_len=[128, 256], chunk_len=[0, 128], Hq=8, Hkv=2, d=64, mask_fn=bern(0.3)),
    "g3_ragged": dict(prefix_len=[0, 448], chunk_len=[200, 129], Hq=6, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g7_d64": dict(prefix_len=[640, 64], chunk_len=[300, 64], Hq=14, Hkv=2, d=64, mask_fn=bern(0.1)),
}


def make_small(name, seed=21):
    kw = dict(SMALL[name])
    return make_workload(name, kw.pop("prefix_len"), kw.pop("chunk_len"), kw.pop("Hq"), kw.pop("Hkv"),
                         kw.pop("d"), "bf16", kw.pop("mask_fn"), seed, **kw)


def split_prefill(dv, w, tables, counts, split_pages, kp=None, vp=None, workspace=None):
    return cpa.chunked_prefill(dv["q"], dv["kp"] if kp is None else kp, dv["vp"] if vp is None else vp,
                               dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                               return_lse=True, split_pages=split_pages, workspace=workspace)


@pytest.mark.parametrize("split", [1, 2, 5])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_split_small(name, split):
    print(f"\n[case] split small {name} split_pages={split}", flush=True)
    w = make_small(name)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    o, lse = split_prefill(dv, w, tables, counts, split)
    torch.cuda.synchronize()
    O, L = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    compare(w, o, O, f"{name} split {split}")
    lg = lse.cpu().numpy().astype(np.float64)
    Lr = L.T
    fin = np.isfinite(Lr)
    assert np.array_equal(np.isfinite(lg), fin)
    if fin.any():
        # bf16 weights (<= 2^-9) and the bf16 rounding of the pre-scaled Q (~1.1e-3 RMS per
        # score, 5 sigma 5.7e-3 when one key dominates a row): the bound of the unsplit path
        assert np.max(np.abs(lg[fin] - Lr[fin])) < 2 ** -7
    if name == "all_zero":
        assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_split_matches_unsplit():
    # same tables, split into 3-page ranges vs one range: equal up to the fp32 partials' rounding
    w = make_small("g4_ragged_multi", seed=5)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    o1, l1 = split_prefill(dv, w, tables, counts, 0)
    o2, l2 = split_prefill(dv, w, tables, counts, 3)
    assert float((o1.float() - o2.float()).abs().max()) <= 2 ** -7
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(l2))
    assert float((l1[fin] - l2[fin]).abs().max()) < 1e-3


def test_split_workspace_reuse():
    # one workspace for two calls in a row, the second smaller: nothing carries over
    wa = make_small("g2_varlen_d128", seed=7)
    wb = make_small("g4_d64", seed=8)
    ws = torch.empty(cpa.split_workspace_bytes(wa.q.shape[0], wa.Hq, wa.d, wa.nkvb_max, 2), dtype=torch.uint8,
                     device="cuda")
    assert cpa.split_workspace_bytes(wb.q.shape[0], wb.Hq, wb.d, wb.nkvb_max, 2) <= ws.numel()
    for w in (wa, wb):
        dv = upload(w)
        tables, counts = gpu_tables(dv, w)
        o, _ = split_prefill(dv, w, tables, counts, 2, workspace=ws)
        T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
        O, _ = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
        compare(w, o, O, f"{w.name} reuse")


def test_split_poison_unselected_pages():
    w = make_small("g4_ragged_multi")
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    keep = np.zeros(w.n_pages, dtype=bool)
    for b in range(w.B):
        for g in range(w.Hkv):
            keep[w.page_map[b, T[b, g, :C[b, g]]]] = True
    kp, vp = w.k_pages.copy(), w.v_pages.copy()
    kp[~keep] = np.nan
    vp[~keep] = np.nan
    o1, l1 = split_prefill(dv, w, tables, counts, 2)
    o2, l2 = split_prefill(dv, w, tables, counts, 2, kp=torch.from_numpy(kp).cuda().to(torch.bfloat16),
                           vp=torch.from_numpy(vp).cuda().to(torch.bfloat16))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["c3s_128k_one_group", "c5b_varlen_independent"])
def test_split_full_size(name):
    print(f"\n[case] split full {name}", flush=True)
    w = make_config(name)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    assert np.array_equal(tables.cpu().numpy(), T) and np.array_equal(counts.cpu().numpy(), C)
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    sp = cpa.plan_split_pages(w.B, w.Hq, w.Hkv, w.max_chunk_len, w.nkvb_max, n_cus)
    if sp == 0:
        sp = 128   # the varlen batch fills the GPU unsplit; split it anyway to test the merge
    o, lse = split_prefill(dv, w, tables, counts, sp)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    S = sample_rows(w, 256, seed=3)
    Os, Ls = oracle.attention_rows(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len,
                                   w.Hkv, S)
    rows = torch.from_numpy(w.cu_q[S[:, 0]] + S[:, 2]).cuda()
    heads = torch.from_numpy(S[:, 1]).cuda()
    compare(w, o[rows, heads].float().cpu().numpy(), Os, f"{name} split {sp}")
    assert np.max(np.abs(lse[rows, heads].cpu().numpy() - Ls)) < 2e-2


@pytest.mark.parametrize("name", ["g4_d64", "g4_ragged_multi"])
def test_auto_split(name):
    # split_pages="auto" runs the range length plan_split_pages gives for this device: the same
    # launch, bit for bit, as passing that length, for bf16 and fp8 pools; fp32 pools (no
    # split-KV form) run unsplit
    print(f"\n[case] auto split {name}", flush=True)
    w = make_small(name)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    sp = cpa.plan_split_pages(w.B, w.Hq, w.Hkv, w.max_chunk_len, tables.shape[-1], n_cus)
    assert sp > 0   # a few tiles on a full GPU: the plan splits
    o1, l1 = split_prefill(dv, w, tables, counts, "auto")
    o2, l2 = split_prefill(dv, w, tables, counts, sp)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    O, L = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    compare(w, o1, O, f"{name} auto split")
    kq = (dv["kp"].float() / 0.5).to(torch.float8_e4m3fn)
    vq = (dv["vp"].float() / 0.5).to(torch.float8_e4m3fn)
    f1 = cpa.chunked_prefill(dv["q"], kq, vq, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                             return_lse=True, split_pages="auto", k_scale=0.5, v_scale=0.5)
    f2 = cpa.chunked_prefill(dv["q"], kq, vq, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                             return_lse=True, split_pages=sp, k_scale=0.5, v_scale=0.5)
    torch.cuda.synchronize()
    assert torch.equal(f1[0], f2[0]) and torch.equal(f1[1], f2[1])
    q32, k32, v32 = dv["q"].float(), dv["kp"].float(), dv["vp"].float()
    g1 = cpa.chunked_prefill(q32, k32, v32, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                             return_lse=True, split_pages="auto")
    g2 = cpa.chunked_prefill(q32, k32, v32, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                             return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1])
