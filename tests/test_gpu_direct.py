"""GPU parity of the direct block-sparse baseline (cpa_build_block_plans +
cpa_chunked_prefill_direct) against the oracle's per-(head, query block) attention.

Plans must match bit for bit; outputs within the bf16 bars of the union path (max-abs 2e-2,
mean-abs 2e-3), LSE within 2^-7.  Pages that no plan selects, and tokens past a sequence's end,
are NaN-poisoned in some cases: they must not change the output.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_reduce_amd as cpa
from workloads import make_config, make_workload
from workloads.configs import mask_all, mask_bernoulli, mask_stripes

from _gpu import compare, sample_rows, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def bern(p, local=1):
    return lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=local)


SMALL = {
    "g4_d64": dict(prefix_len=[768], chunk_len=[256], Hq=8, Hkv=2, d=64, mask_fn=bern(0.1)),
    "g2_varlen_d128": dict(prefix_len=[0, 640, 1280], chunk_len=[320, 192, 64], Hq=4, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g4_ragged_multi": dict(prefix_len=[0, 192, 4096], chunk_len=[37, 130, 255], Hq=8, Hkv=2, d=128, mask_fn=bern(0.05)),
    "g8_d128": dict(prefix_len=[512], chunk_len=[256], Hq=16, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g1_d128": dict(prefix_len=[1024, 64], chunk_len=[192, 100], Hq=2, Hkv=2, d=128, mask_fn=bern(0.3)),
    "g3_d64_noise": dict(prefix_len=[448, 64], chunk_len=[192, 256], Hq=6, Hkv=2, d=64, mask_fn=bern(0.1), noncausal_noise=0.3, mask_values=True),
    "stripes_d128": dict(prefix_len=[1536], chunk_len=[512], Hq=8, Hkv=2, d=128, mask_fn=lambda rng, *a: mask_stripes(rng, *a, p=0.1, shared_per_group=False)),
    "all_zero": dict(prefix_len=[256], chunk_len=[128], Hq=8, Hkv=2, d=128, mask_fn=lambda rng, *a: mask_all(rng, *a, value=0)),
    "zero_len_chunk": dict(prefix_len=[128, 256], chunk_len=[0, 128], Hq=8, Hkv=2, d=64, mask_fn=bern(0.3)),
}


def make_small(name, seed=51):
    kw = dict(SMALL[name])
    return make_workload(name, kw.pop("prefix_len"), kw.pop("chunk_len"), kw.pop("Hq"), kw.pop("Hkv"),
                         kw.pop("d"), "bf16", kw.pop("mask_fn"), seed, **kw)


def run_direct(dv, w, plans, counts, kp=None, vp=None):
    vpd = (dv["vp"] if vp is None else vp).transpose(2, 3).contiguous()
    return cpa.chunked_prefill_direct(dv["q"], dv["kp"] if kp is None else kp, vpd, dv["pm"], plans, counts,
                                      dv["cu"], dv["pl"], w.max_chunk_len, return_lse=True)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_direct_small(name):
    print(f"\n[case] direct {name}", flush=True)
    w = make_small(name)
    dv = upload(w)
    plans, counts = cpa.build_block_plans(dv["masks"], dv["pb"], dv["cb"])
    Pn, Cn = oracle.block_plans(w.masks, w.prefix_blocks, w.chunk_blocks, w.nkvb_max)
    assert np.array_equal(plans.cpu().numpy(), Pn) and np.array_equal(counts.cpu().numpy(), Cn)
    o, lse = run_direct(dv, w, plans, counts)
    torch.cuda.synchronize()
    O, L = oracle.block_sparse_attention(w.q, w.k_pages, w.v_pages, w.page_map, Pn, Cn, w.cu_q, w.prefix_len, w.Hkv)
    compare(w, o, O, f"direct {name}")
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L.T)
    assert np.array_equal(np.isfinite(lg), fin)
    if fin.any():
        assert np.max(np.abs(lg[fin] - L.T[fin])) < 2 ** -7
    if name == "all_zero":
        assert torch.all(o == 0)


def test_direct_poison_unplanned_pages_and_tail_tokens():
    w = make_small("g4_ragged_multi")
    dv = upload(w)
    plans, counts = cpa.build_block_plans(dv["masks"], dv["pb"], dv["cb"])
    Pn, Cn = oracle.block_plans(w.masks, w.prefix_blocks, w.chunk_blocks, w.nkvb_max)
    o1, l1 = run_direct(dv, w, plans, counts)
    keep = np.zeros(w.n_pages, dtype=bool)
    for b in range(w.B):
        for h in range(w.Hq):
            for qi in range(w.nqb_max):
                keep[w.page_map[b, Pn[b, h, qi, :Cn[b, h, qi]]]] = True
    kp, vp = w.k_pages.copy(), w.v_pages.copy()
    kp[~keep] = np.nan
    vp[~keep] = np.nan
    for b in range(w.B):   # and the slots past each sequence's end on its last page
        L = int(w.prefix_len[b] + w.chunk_len[b])
        if L % 64:
            kp[w.page_map[b, L // 64], :, L % 64:] = np.nan
            vp[w.page_map[b, L // 64], :, L % 64:] = np.nan
    o2, l2 = run_direct(dv, w, plans, counts, kp=torch.from_numpy(kp).cuda().to(torch.bfloat16),
                        vp=torch.from_numpy(vp).cuda().to(torch.bfloat16))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["c3_128k_last_chunk", "c5b_varlen_independent"])
def test_direct_full_size(name):
    print(f"\n[case] direct full {name}", flush=True)
    w = make_config(name)
    dv = upload(w)
    plans, counts = cpa.build_block_plans(dv["masks"], dv["pb"], dv["cb"])
    Pn, Cn = oracle.block_plans(w.masks, w.prefix_blocks, w.chunk_blocks, w.nkvb_max)
    assert np.array_equal(plans.cpu().numpy(), Pn) and np.array_equal(counts.cpu().numpy(), Cn)
    o, lse = run_direct(dv, w, plans, counts)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    S = sample_rows(w, 256, seed=9)
    Os, Ls = oracle.block_sparse_rows(w.q, w.k_pages, w.v_pages, w.page_map, Pn, Cn, w.cu_q, w.prefix_len, w.Hkv, S)
    r = torch.from_numpy(w.cu_q[S[:, 0]] + S[:, 2]).cuda()
    h = torch.from_numpy(S[:, 1]).cuda()
    compare(w, o[r, h].float().cpu().numpy(), Os, f"direct {name}")
    assert np.max(np.abs(lse[r, h].cpu().numpy() - Ls)) < 2e-2
