"""GPU parity of dim-major V pages (cpa_chunked_prefill_vt) against the fp64 CPU oracle.

A dim-major pool holds the same values as the token-major one, so the attention is the same:
the oracle takes the token-major pool and the GPU the transposed copy.  The dim-major path sums
the keys of each 16-key step in another order, so it agrees with the token-major path up to
fp32 rounding, which the bf16 output can turn into one unit in the last place at most; the tests
check that bound beside the oracle comparison.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_reduce_amd as cpa
from workloads import make_config, make_workload
from workloads.configs import mask_all, mask_bernoulli, mask_stripes

from _gpu import compare, gpu_tables, sample_rows, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def bern(p, local=1):
    return lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=local)


SMALL = {
    "g4_bf16_d64": dict(prefix_len=[768], chunk_len=[256], Hq=8, Hkv=2, d=64, dtype="bf16", mask_fn=bern(0.05)),
    "g2_varlen_bf16_d128": dict(prefix_len=[0, 640, 1280], chunk_len=[320, 192, 64], Hq=4, Hkv=2, d=128, dtype="bf16", mask_fn=bern(0.1)),
    "g8_bf16_d128": dict(prefix_len=[512], chunk_len=[256], Hq=16, Hkv=2, d=128, dtype="bf16", mask_fn=bern(0.1)),
    "g1_bf16_d128": dict(prefix_len=[1024, 64], chunk_len=[192, 100], Hq=2, Hkv=2, d=128, dtype="bf16", mask_fn=bern(0.3)),
    "g4_bf16_ragged_multi": dict(prefix_len=[0, 192, 4096], chunk_len=[37, 130, 255], Hq=8, Hkv=2, d=128, dtype="bf16", mask_fn=bern(0.05)),
    "g1_f32_d128_ragged": dict(prefix_len=[320, 0], chunk_len=[100, 77], Hq=3, Hkv=3, d=128, dtype="f32", mask_fn=bern(0.2)),
    "g4_f32_d64_stripes": dict(prefix_len=[1536], chunk_len=[512], Hq=8, Hkv=2, d=64, dtype="f32", mask_fn=lambda rng, *a: mask_stripes(rng, *a, p=0.1, shared_per_group=False)),
    "all_zero_bf16": dict(prefix_len=[256], chunk_len=[128], Hq=8, Hkv=2, d=128, dtype="bf16", mask_fn=lambda rng, *a: mask_all(rng, *a, value=0)),
    "zero_len_chunk": dict(prefix_len=[128, 256], chunk_len=[0, 128], Hq=8, Hkv=2, d=64, dtype="bf16", mask_fn=bern(0.3)),
    "g3_bf16_ragged": dict(prefix_len=[0, 448], chunk_len=[200, 129], Hq=6, Hkv=2, d=128, dtype="bf16", mask_fn=bern(0.1)),
    "g7_bf16_d64": dict(prefix_len=[640, 64], chunk_len=[300, 64], Hq=14, Hkv=2, d=64, dtype="bf16", mask_fn=bern(0.1)),
}


def make_small(name, seed=31):
    kw = dict(SMALL[name])
    return make_workload(name, kw.pop("prefix_len"), kw.pop("chunk_len"), kw.pop("Hq"), kw.pop("Hkv"),
                         kw.pop("d"), kw.pop("dtype"), kw.pop("mask_fn"), seed, **kw)


def dim_major(vp):
    """[n_pages][Hkv][64][d] -> contiguous [n_pages][Hkv][d][64]"""
    return vp.transpose(2, 3).contiguous()


def close_to_token_major(o, lse, o_t, lse_t):
    """Within one output ulp (2^-7 relative for bf16) and 1e-4 in the LSE of the token-major run
    (fp32 sums of up to 2^17 terms in another order)."""
    of, otf = o.float(), o_t.float()
    assert bool((torch.isfinite(of) == torch.isfinite(otf)).all())
    diff = (of - otf).abs()
    ulp = 2 ** -7 if o.dtype == torch.bfloat16 else 2 ** -20
    assert bool((diff <= ulp * otf.abs() + 1e-6).all()), f"max diff {float(diff.max()):.3e}"
    fin = torch.isfinite(lse_t)
    assert torch.equal(fin, torch.isfinite(lse))
    if bool(fin.any()):
        assert float((lse[fin] - lse_t[fin]).abs().max()) < 1e-4


def run(dv, w, tables, counts, v_layout, vp=None, kp=None, split_pages=0):
    if vp is None:
        vp = dim_major(dv["vp"]) if v_layout == "dim" else dv["vp"]
    return cpa.chunked_prefill(dv["q"], dv["kp"] if kp is None else kp, vp, dv["pm"], tables, counts, dv["cu"],
                               dv["pl"], w.max_chunk_len, return_lse=True, split_pages=split_pages,
                               v_layout=v_layout)


@pytest.mark.parametrize("split", [0, 2])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_dim_major_small(name, split):
    w = make_small(name)
    print(f"\n[case] dim-major V {name} split_pages={split}", flush=True)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    if split and w.dtype != "bf16":
        # split-KV is bf16 only: a call that would cut the table into ranges is refused, in
        # either V layout, before anything is launched
        assert -(-tables.shape[-1] // split) > 1
        for layout in ("dim", "token"):
            with pytest.raises(cpa.CpaError, match="unsupported"):
                run(dv, w, tables, counts, layout, split_pages=split)
        return
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    o, lse = run(dv, w, tables, counts, "dim", split_pages=split)
    o_t, lse_t = run(dv, w, tables, counts, "token", split_pages=split)
    torch.cuda.synchronize()
    O, L = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    compare(w, o, O, f"{name} dim-major")
    fin = np.isfinite(L.T)
    lg = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isfinite(lg), fin)
    if fin.any():
        assert np.max(np.abs(lg[fin] - L.T[fin])) < (2 ** -7 if w.dtype == "bf16" else 1e-4)
    close_to_token_major(o, lse, o_t, lse_t)


def test_dim_major_tail_tokens_are_not_read():
    # tokens past each sequence's end on its last page hold NaN (in K and in V): neither layout
    # may let them into the output
    w = make_small("g4_bf16_ragged_multi")
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    o1, l1 = run(dv, w, tables, counts, "dim")
    o1t, l1t = run(dv, w, tables, counts, "token")
    kp, vp = w.k_pages.copy(), w.v_pages.copy()
    n = 0
    for b in range(w.B):
        L = int(w.prefix_len[b] + w.chunk_len[b])
        if L % 64:
            ph = w.page_map[b, L // 64]
            kp[ph, :, L % 64:] = np.nan
            vp[ph, :, L % 64:] = np.nan
            n += 1
    assert n >= 2
    dt = dv["q"].dtype
    kpt = torch.from_numpy(kp).cuda().to(dt)
    vpt = torch.from_numpy(vp).cuda().to(dt)
    o2, l2 = run(dv, w, tables, counts, "dim", vp=dim_major(vpt), kp=kpt)
    o3, l3 = run(dv, w, tables, counts, "token", vp=vpt, kp=kpt)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1t, o3) and torch.equal(l1t, l3)


def test_dim_major_strided_view():
    # dim rows padded to 72 tokens: the kernel gets a [n_pages][Hkv][d][64] view with dim stride 72
    w = make_small("g2_varlen_bf16_d128")
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    n_pages, Hkv, _, d = dv["vp"].shape
    padded = torch.full((n_pages, Hkv, d, 72), float("nan"), dtype=dv["vp"].dtype, device="cuda")
    padded[..., :64] = dim_major(dv["vp"])
    view = padded[..., :64]
    assert view.stride(2) == 72
    o1, l1 = run(dv, w, tables, counts, "dim")
    o2, l2 = run(dv, w, tables, counts, "dim", vp=view)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_dim_major_poison_unselected_pages():
    w = make_small("g4_bf16_ragged_multi")
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    keep = np.zeros(w.n_pages, dtype=bool)
    for b in range(w.B):
        for g in range(w.Hkv):
            keep[w.page_map[b, T[b, g, :C[b, g]]]] = True
    vp = w.v_pages.copy()
    vp[~keep] = np.nan
    o1, l1 = run(dv, w, tables, counts, "dim")
    o2, l2 = run(dv, w, tables, counts, "dim", vp=dim_major(torch.from_numpy(vp).cuda().to(torch.bfloat16)))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["c3_128k_last_chunk", "c5b_varlen_independent", "c3s_128k_one_group",
                                  "c3g7_128k_gqa7"])
def test_dim_major_full_size(name):
    print(f"\n[case] dim-major V full {name}", flush=True)
    w = make_config(name)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    sp = 0
    if name.startswith("c3s"):
        n_cus = torch.cuda.get_device_properties(0).multi_processor_count
        sp = cpa.plan_split_pages(w.B, w.Hq, w.Hkv, w.max_chunk_len, w.nkvb_max, n_cus)
    o, lse = run(dv, w, tables, counts, "dim", split_pages=sp)
    o_t, lse_t = run(dv, w, tables, counts, "token", split_pages=sp)
    torch.cuda.synchronize()
    close_to_token_major(o, lse, o_t, lse_t)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    S = sample_rows(w, 256, seed=5)
    Os, Ls = oracle.attention_rows(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len,
                                   w.Hkv, S)
    rows = torch.from_numpy(w.cu_q[S[:, 0]] + S[:, 2]).cuda()
    heads = torch.from_numpy(S[:, 1]).cuda()
    compare(w, o[rows, heads].float().cpu().numpy(), Os, f"{name} dim-major")
    assert np.max(np.abs(lse[rows, heads].cpu().numpy() - Ls)) < 2e-2
