"""The chunked-prefill loop end to end: one sequence prefilled chunk after chunk against a paged
cache that starts as NaN everywhere.  Each chunk appends its own K/V rows (cpa_append_kv), builds
its tables from its own masks and runs the prefill; the output must match the oracle run on the
complete pools, since the causal rule hides every position a later chunk writes and the slots
past the sequence's end on its last page are never written at all.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_reduce_amd as cpa
from workloads import make_workload
from workloads.configs import mask_bernoulli

from _gpu import compare

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# every chunk but the last is whole pages (the next chunk's prefix is a multiple of 64); the last
# one ends inside a page
CHUNKS = [256, 64, 192, 320, 100]


def bern(p):
    return lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=1)


@pytest.mark.parametrize("v_layout,d,split", [("token", 64, 0), ("dim", 128, 0), ("dim", 128, 3)])
def test_sequence_prefilled_chunk_by_chunk(v_layout, d, split):
    print(f"\n[case] lifecycle {v_layout} d{d} split{split}", flush=True)
    total = sum(CHUNKS)
    full = make_workload("seq", [0], [total], 8, 2, d, "bf16", bern(0.3), 91)
    kv = (full.k_pages, full.v_pages, full.page_map, full.poison_page)
    pm = torch.from_numpy(full.page_map).cuda()
    kp = torch.full(full.k_pages.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    n_pages, hkv = full.k_pages.shape[:2]
    vshape = (n_pages, hkv, 64, d) if v_layout == "token" else (n_pages, hkv, d, 64)
    vp = torch.full(vshape, float("nan"), dtype=torch.bfloat16, device="cuda")
    seeds = np.random.default_rng(3).integers(1 << 30, size=len(CHUNKS))
    start = 0
    for k, n in enumerate(CHUNKS):
        pos = np.arange(start, start + n)
        ph, sl = full.page_map[0, pos // 64], pos % 64
        krows = torch.from_numpy(full.k_pages[ph, :, sl]).to(torch.bfloat16).contiguous().cuda()
        vrows = torch.from_numpy(full.v_pages[ph, :, sl]).to(torch.bfloat16).contiguous().cuda()
        cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        pl = torch.tensor([start], dtype=torch.int32, device="cuda")
        cpa.append_kv(krows, vrows, kp, vp, pm, cu, pl, n, v_layout=v_layout)

        w = make_workload(f"chunk{k}", [start], [n], 8, 2, d, "bf16", bern(0.3), int(seeds[k]), kv=kv)
        masks = torch.from_numpy(np.ascontiguousarray(w.masks)).cuda()
        tables, counts = cpa.build_block_tables(masks, torch.from_numpy(w.prefix_blocks).cuda(),
                                                torch.from_numpy(w.chunk_blocks).cuda(), w.Hkv)
        T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
        assert np.array_equal(tables.cpu().numpy(), T) and np.array_equal(counts.cpu().numpy(), C)
        q = torch.from_numpy(w.q).to(torch.bfloat16).cuda()
        o, lse = cpa.chunked_prefill(q, kp, vp, pm, tables, counts, cu, pl, n, return_lse=True,
                                     v_layout=v_layout, split_pages=split)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(o).all()), f"chunk {k}: a slot that holds no token was read"
        O, L = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
        compare(w, o, O, f"chunk {k} at {start}")
        assert np.max(np.abs(lse.cpu().numpy() - L.T)) < 2e-2
        start += n

    # the cache now holds exactly the sequence's rows; everything else is still NaN
    pages = torch.from_numpy(full.page_map[0, : (total + 63) // 64].astype(np.int64)).cuda()
    kref = torch.from_numpy(full.k_pages).to(torch.bfloat16).cuda()
    vref = torch.from_numpy(full.v_pages).to(torch.bfloat16).cuda()
    got_v = vp.transpose(2, 3) if v_layout == "dim" else vp
    last = total // 64
    whole = pages[:last]
    assert torch.equal(kp[whole], kref[whole]) and torch.equal(got_v[whole], vref[whole])
    tail = total % 64
    assert torch.equal(kp[pages[last], :, :tail], kref[pages[last], :, :tail])
    assert torch.equal(got_v[pages[last], :, :tail], vref[pages[last], :, :tail])
    assert bool(torch.isnan(kp[pages[last], :, tail:].float()).all())
    assert bool(torch.isnan(got_v[pages[last], :, tail:].float()).all())
    others = torch.ones(n_pages, dtype=torch.bool, device="cuda")
    others[pages] = False
    assert bool(torch.isnan(kp[others].float()).all()) and bool(torch.isnan(got_v[others].float()).all())


def test_max_chunk_len_read_from_cu_q():
    """Leaving max_chunk_len out makes the binding read the longest chunk from cu_q: every entry
    point that takes it returns the same bits as when it is passed."""
    print("\n[case] max_chunk_len read from cu_q", flush=True)
    from _gpu import upload
    w = make_workload("mcl", [128, 0, 640], [100, 256, 64], 8, 2, 64, "bf16", bern(0.4), 17)
    dv = upload(w)
    vdim = dv["vp"].transpose(2, 3).contiguous()
    tables, counts = cpa.build_block_tables(dv["masks"], dv["pb"], dv["cb"], w.Hkv)
    args = (dv["q"], dv["kp"])
    for layout, vp in (("token", dv["vp"]), ("dim", vdim)):
        unsplit = None
        for split in (0, 2):
            o1, l1 = cpa.chunked_prefill(*args, vp, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                                         return_lse=True, v_layout=layout, split_pages=split)
            o2, l2 = cpa.chunked_prefill(*args, vp, dv["pm"], tables, counts, dv["cu"], dv["pl"], return_lse=True,
                                         v_layout=layout, split_pages=split)
            assert torch.equal(o1, o2) and torch.equal(l1, l2), (layout, split)
            if split == 0:
                unsplit = o1
        f1, _ = cpa.chunked_prefill_fused(*args, vp, dv["pm"], dv["masks"], dv["cu"], dv["pl"], w.max_chunk_len,
                                          v_layout=layout)
        f2, _ = cpa.chunked_prefill_fused(*args, vp, dv["pm"], dv["masks"], dv["cu"], dv["pl"], v_layout=layout)
        assert torch.equal(f1, f2) and torch.equal(f1, unsplit), layout
    plans, plan_counts = cpa.build_block_plans(dv["masks"], dv["pb"], dv["cb"])
    d1, _ = cpa.chunked_prefill_direct(*args, vdim, dv["pm"], plans, plan_counts, dv["cu"], dv["pl"], w.max_chunk_len)
    d2, _ = cpa.chunked_prefill_direct(*args, vdim, dv["pm"], plans, plan_counts, dv["cu"], dv["pl"])
    assert torch.equal(d1, d2)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    rows = torch.randn((dv["q"].shape[0], w.Hkv, w.d), generator=g, device="cuda").to(torch.bfloat16)
    pools = []
    for mcl in (w.max_chunk_len, None):
        kp, vp = dv["kp"].clone(), dv["vp"].clone()
        cpa.append_kv(rows, rows, kp, vp, dv["pm"], dv["cu"], dv["pl"], mcl)
        pools.append((kp, vp))
    assert torch.equal(pools[0][0], pools[1][0]) and torch.equal(pools[0][1], pools[1][1])
    assert not torch.equal(pools[0][0], dv["kp"])   # the rows did land
