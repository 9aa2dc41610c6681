"""GPU parity at the limits: the largest KV extent the table build takes (65536 blocks, a
4M-token context) and the largest query groups (G = 16, 32), against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_reduce_amd as cpa
from workloads import make_workload
from workloads.configs import mask_bernoulli, mask_stripes

from _gpu import compare, gpu_tables, sample_rows, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MAX_BLOCKS = 65536


@pytest.fixture(scope="module")
def longest():
    # one sequence whose last 128-token chunk ends at block 65535: 4,194,304 tokens of context
    P = (MAX_BLOCKS - 2) * 64
    return make_workload("max_context", [P], [128], 4, 1, 64, "bf16",
                         lambda rng, *a: mask_stripes(rng, *a, p=0.05, shared_per_group=False), 71)


def test_max_context_tables(longest):
    w = longest
    assert w.nkvb_max == MAX_BLOCKS
    dv = upload(w)
    t, c = gpu_tables(dv, w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    assert np.array_equal(t.cpu().numpy(), T) and np.array_equal(c.cpu().numpy(), C)
    assert C[0, 0] > 10000   # thousands of pages: the page-id window is reloaded many times


@pytest.mark.parametrize("mode", ["token", "dim", "split"])
def test_max_context_prefill(longest, mode):
    print(f"\n[case] max context {mode}", flush=True)
    w = longest
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    if mode == "split":
        o, lse = cpa.chunked_prefill(dv["q"], dv["kp"], dv["vp"], dv["pm"], tables, counts, dv["cu"], dv["pl"],
                                     w.max_chunk_len, return_lse=True, split_pages=4096)
    else:
        vp = dv["vp"].transpose(2, 3).contiguous() if mode == "dim" else dv["vp"]
        o, lse = cpa.chunked_prefill(dv["q"], dv["kp"], vp, dv["pm"], tables, counts, dv["cu"], dv["pl"],
                                     w.max_chunk_len, return_lse=True, v_layout=mode)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    S = sample_rows(w, 48, seed=2)
    Os, Ls = oracle.attention_rows(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv, S)
    r = torch.from_numpy(w.cu_q[S[:, 0]] + S[:, 2]).cuda()
    h = torch.from_numpy(S[:, 1]).cuda()
    compare(w, o[r, h].float().cpu().numpy(), Os, f"max context {mode}")
    assert np.max(np.abs(lse[r, h].cpu().numpy() - Ls)) < 2e-2


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 1, 128), (32, 2, 64), (16, 1, 64)])
def test_large_groups(Hq, Hkv, d):
    print(f"\n[case] G = {Hq // Hkv}, d = {d}", flush=True)
    w = make_workload(f"g{Hq // Hkv}", [512, 1024], [192, 77], Hq, Hkv, d, "bf16",
                      lambda rng, *a: mask_bernoulli(rng, *a, p=0.1, local=1), 72)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    assert np.array_equal(tables.cpu().numpy(), T)
    O, L = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    for v_layout, split in (("token", 0), ("dim", 0), ("token", 4), ("dim", 4)):
        vp = dv["vp"].transpose(2, 3).contiguous() if v_layout == "dim" else dv["vp"]
        o, lse = cpa.chunked_prefill(dv["q"], dv["kp"], vp, dv["pm"], tables, counts, dv["cu"], dv["pl"],
                                     w.max_chunk_len, return_lse=True, v_layout=v_layout, split_pages=split)
        torch.cuda.synchronize()
        compare(w, o, O, f"G={Hq // Hkv} {v_layout} split {split}")
        assert np.max(np.abs(lse.cpu().numpy() - L.T)) < 2 ** -7


WIDE = (1 << 24) + 64   # row stride in elements: past the direct-to-LDS kernel's 32-bit offsets


def wide_view(x, elem):
    """x [n][H][R][C] (R = 64 tokens, or d dim rows for dim-major V) as a CUDA view with row stride
    WIDE elements and the usual nesting (head stride R * WIDE, page stride H * R * WIDE): a pool
    of n * H * R * WIDE elements of which only the rows' first C are written and read."""
    n, H, R, C = x.shape
    buf = torch.empty((n * H * R - 1) * WIDE + C, dtype=elem, device="cuda")
    v = torch.as_strided(buf, (n, H, R, C), (H * R * WIDE, R * WIDE, WIDE, 1))
    v.copy_(x.cuda())
    return v


@pytest.mark.parametrize("kind,v_layout", [("bf16", "token"), ("bf16", "dim"), ("fp8", "token"), ("fp8", "dim")])
def test_wide_row_stride_pools(kind, v_layout):
    # pools whose offsets within a page overflow 32 bits (and whose page offsets reach 2^32
    # bytes) go through the register-staged kernel; same bars against the oracle.  One KV group,
    # two KV blocks (the second partial), three pages: 3 * 64 * WIDE elements per tensor.
    print(f"\n[case] wide row stride {kind} {v_layout}", flush=True)
    w = make_workload("wide", [0], [100], 4, 1, 64, "bf16",
                      lambda rng, *a: mask_bernoulli(rng, *a, p=0.5, local=1), 73)
    assert w.n_pages == 3
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    if kind == "bf16":
        kt = torch.from_numpy(w.k_pages).to(torch.bfloat16)
        vt = torch.from_numpy(w.v_pages).to(torch.bfloat16)
        kdq, vdq, ks, vs, elem = w.k_pages, w.v_pages, 1.0, 1.0, torch.bfloat16
    else:
        ks, vs = 0.37, 1.9
        kt = (torch.from_numpy(w.k_pages) / ks).to(torch.float8_e4m3fn).view(torch.uint8)
        vt = (torch.from_numpy(w.v_pages) / vs).to(torch.float8_e4m3fn).view(torch.uint8)
        kdq, vdq = oracle.dequant_e4m3(kt.numpy(), ks), oracle.dequant_e4m3(vt.numpy(), vs)
        elem = torch.uint8
    if v_layout == "dim":
        vt = vt.transpose(2, 3).contiguous()
    kw, vw = wide_view(kt, elem), wide_view(vt, elem)
    if kind == "fp8":
        kw, vw = kw.view(torch.float8_e4m3fn), vw.view(torch.float8_e4m3fn)
    o, lse = cpa.chunked_prefill(dv["q"], kw, vw, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                                 return_lse=True, v_layout=v_layout, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    O, L = oracle.paged_attention(w.q, kdq, vdq, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    compare(w, o, O, f"wide {kind} {v_layout}")
    assert np.max(np.abs(lse.cpu().numpy() - L.T)) < 2e-2
    del kw, vw
    torch.cuda.empty_cache()
