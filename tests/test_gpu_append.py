"""GPU parity of the KV append (cpa_append_kv) against the CPU oracle: bit-exact pools.

The append is a copy, so the GPU's pools must equal the oracle's bit for bit, in both V layouts,
including the slots it must leave alone (the rest of a partial last page, pages it cannot
resolve).  The end-to-end case appends a chunk whose K/V slots were poisoned and then runs the
tables and the prefill over the result.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_reduce_amd as cpa
from workloads import make_config, make_workload
from workloads.configs import mask_bernoulli

from _gpu import compare, gpu_tables, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def bern(p, local=1):
    return lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=local)


CASES = {
    "bf16_d128_ragged": dict(prefix_len=[0, 192, 4096], chunk_len=[37, 130, 255], Hq=8, Hkv=2, d=128, dtype="bf16"),
    "bf16_d64_aligned": dict(prefix_len=[768], chunk_len=[256], Hq=8, Hkv=2, d=64, dtype="bf16"),
    "f32_d128_ragged": dict(prefix_len=[320, 0], chunk_len=[100, 77], Hq=3, Hkv=3, d=128, dtype="f32"),
    "f32_d64_zero_chunk": dict(prefix_len=[128, 256], chunk_len=[0, 70], Hq=8, Hkv=4, d=64, dtype="f32"),
}


def make(name, seed=41):
    kw = dict(CASES[name])
    return make_workload(name, kw.pop("prefix_len"), kw.pop("chunk_len"), kw.pop("Hq"), kw.pop("Hkv"),
                         kw.pop("d"), kw.pop("dtype"), bern(0.2), seed)


def chunk_rows(w, pages):
    """The chunk's K (or V) rows [Tq][Hkv][d] as they sit in the workload's pools."""
    rows = []
    for b in range(w.B):
        pos = w.prefix_len[b] + np.arange(w.chunk_len[b])
        rows.append(pages[w.page_map[b, pos // 64], :, pos % 64])
    return np.concatenate(rows, axis=0) if rows else np.zeros((0, w.Hkv, w.d))


@pytest.mark.parametrize("v_layout", ["token", "dim"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_append_matches_oracle(name, v_layout):
    print(f"\n[case] append {name} {v_layout}", flush=True)
    w = make(name)
    rng = np.random.default_rng(5)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Tq = int(w.chunk_len.sum())
    k_new = torch.from_numpy(rng.standard_normal((Tq, w.Hkv, w.d)).astype(np.float32)).to(dt)
    v_new = torch.from_numpy(rng.standard_normal((Tq, w.Hkv, w.d)).astype(np.float32)).to(dt)
    pm = w.page_map.copy()
    if w.B > 1 and w.chunk_len[-1] > 64:   # one page that cannot be resolved: its rows stay out
        pm[-1, (w.prefix_len[-1] + 64) // 64] = w.n_pages + 3
    kp = torch.from_numpy(w.k_pages).to(dt).cuda()
    vp = torch.from_numpy(w.v_pages).to(dt).cuda()
    vpl = vp.transpose(2, 3).contiguous() if v_layout == "dim" else vp.clone()
    cpa.append_kv(k_new.cuda(), v_new.cuda(), kp, vpl, torch.from_numpy(pm).cuda(), torch.from_numpy(w.cu_q).cuda(),
                  torch.from_numpy(w.prefix_len).cuda(), w.max_chunk_len, v_layout=v_layout)
    torch.cuda.synchronize()
    # the oracle on the same (already rounded) values, compared as raw bits
    K, V = oracle.append_kv(k_new.float().numpy(), v_new.float().numpy(),
                            torch.from_numpy(w.k_pages).to(dt).float().numpy(),
                            torch.from_numpy(w.v_pages).to(dt).float().numpy(), pm, w.cu_q, w.prefix_len)
    got_v = vpl.transpose(2, 3) if v_layout == "dim" else vpl
    assert torch.equal(kp.cpu(), torch.from_numpy(K).to(dt)), "K pool differs"
    assert torch.equal(got_v.cpu(), torch.from_numpy(V).to(dt)), "V pool differs"


@pytest.mark.parametrize("v_layout", ["token", "dim"])
def test_append_then_prefill(v_layout):
    # the chunk's own K/V slots start as NaN; appending the chunk rows restores the workload's
    # pools exactly, and the tables and the prefill then match the oracle
    w = make_workload("e2e", [0, 192, 4096], [37, 130, 255], 8, 2, 128, "bf16", bern(0.05), 9)
    dv = upload(w)
    k_rows = torch.from_numpy(chunk_rows(w, w.k_pages)).cuda().to(torch.bfloat16)
    v_rows = torch.from_numpy(chunk_rows(w, w.v_pages)).cuda().to(torch.bfloat16)
    kp = dv["kp"].clone()
    vp = dv["vp"].clone()
    for b in range(w.B):
        pos = w.prefix_len[b] + np.arange(w.chunk_len[b])
        pg = torch.from_numpy(w.page_map[b, pos // 64].astype(np.int64)).cuda()
        sl = torch.from_numpy((pos % 64).astype(np.int64)).cuda()
        kp[pg, :, sl] = float("nan")
        vp[pg, :, sl] = float("nan")
    vpl = vp.transpose(2, 3).contiguous() if v_layout == "dim" else vp
    cpa.append_kv(k_rows, v_rows, kp, vpl, dv["pm"], dv["cu"], dv["pl"], w.max_chunk_len, v_layout=v_layout)
    got_v = vpl.transpose(2, 3) if v_layout == "dim" else vpl
    assert torch.equal(kp, dv["kp"]) and torch.equal(got_v, dv["vp"])
    tables, counts = gpu_tables(dv, w)
    o, _ = cpa.chunked_prefill(dv["q"], kp, vpl, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                               v_layout=v_layout)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    O, _ = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    compare(w, o, O, f"append+prefill {v_layout}")


@pytest.mark.parametrize("v_layout", ["token", "dim"])
def test_append_full_size_chunk(v_layout):
    # the 2048-row chunk of the 128K workload into its 32 pages of every group
    print(f"\n[case] append full c3 {v_layout}", flush=True)
    w = make_config("c3_128k_last_chunk")
    dv = upload(w)
    k_rows = torch.from_numpy(chunk_rows(w, w.k_pages)).cuda().to(torch.bfloat16)
    v_rows = torch.from_numpy(chunk_rows(w, w.v_pages)).cuda().to(torch.bfloat16)
    kp = torch.zeros_like(dv["kp"])
    vp = torch.zeros_like(dv["vp"])
    vpl = vp.transpose(2, 3).contiguous() if v_layout == "dim" else vp
    cpa.append_kv(k_rows, v_rows, kp, vpl, dv["pm"], dv["cu"], dv["pl"], w.max_chunk_len, v_layout=v_layout)
    torch.cuda.synchronize()
    pages = torch.from_numpy(w.page_map[0, w.prefix_len[0] // 64:].astype(np.int64)).cuda()
    got_v = vpl.transpose(2, 3) if v_layout == "dim" else vpl
    assert torch.equal(kp[pages], dv["kp"][pages]) and torch.equal(got_v[pages], dv["vp"][pages])
    others = torch.ones(kp.shape[0], dtype=torch.bool, device="cuda")
    others[pages] = False
    assert not bool(kp[others].any()) and not bool(got_v[others].any())
