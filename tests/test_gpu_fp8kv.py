"""GPU parity of the fp8 KV path (cpa_chunked_prefill_fp8kv) against the fp64 oracle.

The pools hold OCP e4m3 codes; the oracle attends over its own dequantization of the same codes,
decode(x) * scale, so the bars are those of the bf16 path.  Both V layouts run the direct-to-LDS
kernel (codes staged in LDS, each page converted to bf16 once per workgroup; token-major V through
transposed byte reads), unsplit and split-KV.  The append of fp8 rows is checked bit for bit.
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

KS, VS = 0.37, 1.9   # dequantization scales


def bern(p, local=1):
    return lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=local)


SMALL = {
    "g4_d64": dict(prefix_len=[768], chunk_len=[256], Hq=8, Hkv=2, d=64, mask_fn=bern(0.1)),
    "g2_varlen_d128": dict(prefix_len=[0, 640, 1280], chunk_len=[320, 192, 64], Hq=4, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g4_ragged_multi": dict(prefix_len=[0, 192, 4096], chunk_len=[37, 130, 255], Hq=8, Hkv=2, d=128, mask_fn=bern(0.05)),
    "g8_d128": dict(prefix_len=[512], chunk_len=[256], Hq=16, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g16_d64_ragged": dict(prefix_len=[1024], chunk_len=[150], Hq=32, Hkv=2, d=64, mask_fn=bern(0.2)),
    "g1_d128": dict(prefix_len=[1024, 64], chunk_len=[192, 100], Hq=2, Hkv=2, d=128, mask_fn=bern(0.3)),
    "all_zero": dict(prefix_len=[256], chunk_len=[128], Hq=8, Hkv=2, d=128, mask_fn=lambda rng, *a: mask_all(rng, *a, value=0)),
    "zero_len_chunk": dict(prefix_len=[128, 256], chunk_len=[0, 128], Hq=8, Hkv=2, d=64, mask_fn=bern(0.3)),
    "g3_ragged": dict(prefix_len=[0, 448], chunk_len=[200, 129], Hq=6, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g7_d64": dict(prefix_len=[640, 64], chunk_len=[300, 64], Hq=14, Hkv=2, d=64, mask_fn=bern(0.1)),
}


def codes_of(pages, scale):
    """e4m3 codes (uint8) of pages / scale, as a cache writer would store them."""
    return (torch.from_numpy(pages) / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fp8_setup(w):
    kc, vc = codes_of(w.k_pages, KS), codes_of(w.v_pages, VS)
    kdq, vdq = oracle.dequant_e4m3(kc, KS), oracle.dequant_e4m3(vc, VS)
    return kc, vc, kdq, vdq


def run(dv, w, tables, counts, kc, vc, v_layout, split_pages=0):
    k8 = torch.from_numpy(kc).cuda().view(torch.float8_e4m3fn)
    v8 = torch.from_numpy(vc).cuda().view(torch.float8_e4m3fn)
    if v_layout == "dim":
        v8 = v8.view(torch.uint8).transpose(2, 3).contiguous().view(torch.float8_e4m3fn)
    return cpa.chunked_prefill(dv["q"], k8, v8, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                               return_lse=True, v_layout=v_layout, k_scale=KS, v_scale=VS, split_pages=split_pages)


@pytest.mark.parametrize("v_layout", ["token", "dim"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_fp8kv_small(name, v_layout):
    print(f"\n[case] fp8 kv {name} {v_layout}", flush=True)
    kw = dict(SMALL[name])
    w = make_workload(name, kw.pop("prefix_len"), kw.pop("chunk_len"), kw.pop("Hq"), kw.pop("Hkv"), kw.pop("d"),
                      "bf16", kw.pop("mask_fn"), 61, **kw)
    kc, vc, kdq, vdq = fp8_setup(w)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    o, lse = run(dv, w, tables, counts, kc, vc, v_layout)
    torch.cuda.synchronize()
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    O, L = oracle.paged_attention(w.q, kdq, vdq, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    compare(w, o, O, f"fp8 {name} {v_layout}")
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L.T)
    assert np.array_equal(np.isfinite(lg), fin)
    if fin.any():
        assert np.max(np.abs(lg[fin] - L.T[fin])) < 2 ** -7


@pytest.mark.parametrize("split", [1, 3])
@pytest.mark.parametrize("v_layout", ["token", "dim"])
@pytest.mark.parametrize("name", ["g2_varlen_d128", "g4_ragged_multi", "g16_d64_ragged", "g3_ragged", "all_zero",
                                  "zero_len_chunk"])
def test_fp8kv_split_small(name, v_layout, split):
    # split-KV over fp8 pages: every range's partial carries the V scale and the merge is the
    # bf16 path's; ranges of 1 page leave many ranges empty, which must weigh nothing
    print(f"\n[case] fp8 kv split {name} {v_layout} {split}", flush=True)
    kw = dict(SMALL[name])
    w = make_workload(name, kw.pop("prefix_len"), kw.pop("chunk_len"), kw.pop("Hq"), kw.pop("Hkv"), kw.pop("d"),
                      "bf16", kw.pop("mask_fn"), 61, **kw)
    kc, vc, kdq, vdq = fp8_setup(w)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    o, lse = run(dv, w, tables, counts, kc, vc, v_layout, split_pages=split)
    o1, _ = run(dv, w, tables, counts, kc, vc, v_layout)
    torch.cuda.synchronize()
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    O, L = oracle.paged_attention(w.q, kdq, vdq, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    compare(w, o, O, f"fp8 split {name} {v_layout} {split}")
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L.T)
    assert np.array_equal(np.isfinite(lg), fin)
    if fin.any():
        assert np.max(np.abs(lg[fin] - L.T[fin])) < 2 ** -7
    # the unsplit launch on the same codes: the same attention up to the partials' rounding
    assert float((o.float() - o1.float()).abs().max()) <= 2 ** -7


@pytest.mark.parametrize("v_layout", ["token", "dim"])
def test_fp8kv_split_full_size_one_group(v_layout):
    # one KV group of the 128K last chunk (the per-GPU share of an 8-way head split) over fp8
    # pages, split for this device's CUs; sampled rows reach every tile
    print(f"\n[case] fp8 kv split full c3s {v_layout}", flush=True)
    w = make_config("c3s_128k_one_group")
    kc, vc, kdq, vdq = fp8_setup(w)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    sp = cpa.plan_split_pages(w.B, w.Hq, w.Hkv, w.max_chunk_len, w.nkvb_max, n_cus)
    assert sp > 0
    o, lse = run(dv, w, tables, counts, kc, vc, v_layout, split_pages=sp)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    S = sample_rows(w, 256, seed=12)
    Os, Ls = oracle.attention_rows(w.q, kdq, vdq, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv, S)
    r = torch.from_numpy(w.cu_q[S[:, 0]] + S[:, 2]).cuda()
    h = torch.from_numpy(S[:, 1]).cuda()
    compare(w, o[r, h].float().cpu().numpy(), Os, f"fp8 c3s split {sp} {v_layout}")
    assert np.max(np.abs(lse[r, h].cpu().numpy() - Ls)) < 2e-2


@pytest.mark.parametrize("v_layout", ["token", "dim"])
def test_fp8kv_poison_unselected_pages_and_tail_tokens(v_layout):
    w = make_workload("p", [0, 192, 4096], [37, 130, 255], 8, 2, 128, "bf16", bern(0.05), 62)
    kc, vc, _, _ = fp8_setup(w)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    o1, l1 = run(dv, w, tables, counts, kc, vc, v_layout)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    keep = np.zeros(w.n_pages, dtype=bool)
    for b in range(w.B):
        for g in range(w.Hkv):
            keep[w.page_map[b, T[b, g, :C[b, g]]]] = True
    kp, vp = kc.copy(), vc.copy()
    kp[~keep] = 0x7F   # e4m3 NaN
    vp[~keep] = 0x7F
    for b in range(w.B):
        L = int(w.prefix_len[b] + w.chunk_len[b])
        if L % 64:
            kp[w.page_map[b, L // 64], :, L % 64:] = 0x7F
            vp[w.page_map[b, L // 64], :, L % 64:] = 0x7F
    o2, l2 = run(dv, w, tables, counts, kp, vp, v_layout)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("v_layout", ["token", "dim"])
def test_fp8kv_full_size_128k(v_layout):
    print(f"\n[case] fp8 kv full c3 {v_layout}", flush=True)
    w = make_config("c3_128k_last_chunk")
    kc, vc, kdq, vdq = fp8_setup(w)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    o, lse = run(dv, w, tables, counts, kc, vc, v_layout)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    S = sample_rows(w, 256, seed=11)
    Os, Ls = oracle.attention_rows(w.q, kdq, vdq, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv, S)
    r = torch.from_numpy(w.cu_q[S[:, 0]] + S[:, 2]).cuda()
    h = torch.from_numpy(S[:, 1]).cuda()
    compare(w, o[r, h].float().cpu().numpy(), Os, f"fp8 c3 {v_layout}")
    assert np.max(np.abs(lse[r, h].cpu().numpy() - Ls)) < 2e-2


@pytest.mark.parametrize("v_layout", ["token", "dim"])
def test_fp8_append_bit_exact(v_layout):
    w = make_workload("a8", [0, 192, 4096], [37, 130, 255], 8, 2, 128, "bf16", bern(0.05), 63)
    kc, vc, _, _ = fp8_setup(w)
    rng = np.random.default_rng(8)
    Tq = int(w.chunk_len.sum())
    kn = rng.integers(0, 256, (Tq, w.Hkv, w.d), dtype=np.uint8)
    vn = rng.integers(0, 256, (Tq, w.Hkv, w.d), dtype=np.uint8)
    K, V = oracle.append_kv(kn, vn, kc, vc, w.page_map, w.cu_q, w.prefix_len)
    f8 = torch.float8_e4m3fn
    kp = torch.from_numpy(kc).cuda().view(f8)
    vp = torch.from_numpy(vc).cuda()
    vp = (vp.transpose(2, 3).contiguous() if v_layout == "dim" else vp).view(f8)
    cpa.append_kv(torch.from_numpy(kn).cuda().view(f8), torch.from_numpy(vn).cuda().view(f8), kp, vp,
                  torch.from_numpy(w.page_map).cuda(), torch.from_numpy(w.cu_q).cuda(),
                  torch.from_numpy(w.prefix_len).cuda(), w.max_chunk_len, v_layout=v_layout)
    torch.cuda.synchronize()
    got_v = vp.view(torch.uint8)
    got_v = got_v.transpose(2, 3) if v_layout == "dim" else got_v
    assert np.array_equal(kp.view(torch.uint8).cpu().numpy(), K)
    assert np.array_equal(got_v.cpu().numpy(), V)


@pytest.mark.parametrize("kv", ["bf16-dim", "fp8-token", "fp8-dim"])
def test_out_of_range_page_id_reads_as_nan(kv):
    # a block that only group 1 selects gets a page id outside the pool: group 1's heads turn NaN
    # exactly on the rows that reach the block, group 0 is unaffected
    w = make_workload("oor", [768], [256], 8, 2, 64, "bf16", bern(0.05), 64)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    only1 = sorted(set(T[0, 1, :C[0, 1]].tolist()) - set(T[0, 0, :C[0, 0]].tolist()))
    assert only1, "need a block selected by group 1 only"
    kb = only1[0]
    pm = w.page_map.copy()
    pm[0, kb] = w.n_pages + 5
    dv = upload(w, page_map=pm)
    tables, counts = gpu_tables(dv, w)
    dtype, layout = kv.split("-")
    if dtype == "fp8":
        kc, vc, kdq, vdq = fp8_setup(w)
        o, _ = run(dv, w, tables, counts, kc, vc, layout)
    else:
        kdq, vdq = w.k_pages, w.v_pages
        o, _ = cpa.chunked_prefill(dv["q"], dv["kp"], dv["vp"].transpose(2, 3).contiguous(), dv["pm"], tables, counts,
                                   dv["cu"], dv["pl"], w.max_chunk_len, return_lse=True, v_layout="dim")
    torch.cuda.synchronize()
    on = o.float().cpu().numpy()
    seeing = np.arange(int(w.chunk_len[0])) + int(w.prefix_len[0]) >= 64 * kb
    assert np.all(np.isnan(on[seeing][:, 4:8])) and not np.any(np.isnan(on[~seeing][:, 4:8]))
    O, _ = oracle.paged_attention(w.q, kdq, vdq, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    compare(w, o[:, :4], O[:, :4], f"{kv}: group 0 unaffected")


@pytest.mark.parametrize("v_layout", ["token", "dim"])
def test_fp8kv_d64_past_the_id_window(v_layout):
    # d = 64 with tables of ~640 pages: the fp8 pipeline copies one page further ahead, so its
    # page-id window is refilled at another iteration than the bf16 one; every row checked
    print(f"\n[case] fp8 kv d64 long {v_layout}", flush=True)
    w = make_workload("long64", [40960], [192], 8, 2, 64, "bf16", bern(0.9), 63)
    kc, vc, kdq, vdq = fp8_setup(w)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    assert int(C.min()) > 600
    o, lse = run(dv, w, tables, counts, kc, vc, v_layout)
    torch.cuda.synchronize()
    O, L = oracle.paged_attention(w.q, kdq, vdq, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    compare(w, o, O, f"fp8 d64 long {v_layout}")
    assert np.max(np.abs(lse.cpu().numpy() - L.T)) < 2 ** -7
