"""The entry points capture into a HIP graph: they only launch kernels on the caller's stream
(no allocation, no synchronisation, no memset).  A captured table build + prefill replays
several times, with eager work on the GPU in between, and every replay equals the eager result
bit for bit."""
import numpy as np
import pytest
import torch

import sparse_attention_long_reduce_amd as cpa
from workloads import make_workload
from workloads.configs import mask_bernoulli, pack_mask_bits

from _gpu import upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def bern(p, local=1):
    return lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=local)


@pytest.mark.parametrize("mode", ["plain", "split", "dim", "bits", "fp8_token", "fp8_dim", "fp8_split", "fused_token",
                                  "fused_dim", "fused_fp8"])
def test_capture_and_replay(mode):
    w = make_workload("graph", [0, 192, 4096], [37, 130, 255], 8, 2, 128, "bf16", bern(0.05), 81)
    dv = upload(w)
    kp = dv["kp"]
    vp = dv["vp"]
    fp8 = mode.startswith("fp8") or mode == "fused_fp8"
    if fp8:   # e4m3 copies of the pools, scale 1/4
        kp = (kp.float() * 4).to(torch.float8_e4m3fn)
        vp = (vp.float() * 4).to(torch.float8_e4m3fn)
    layout = "dim" if mode in ("dim", "fp8_dim", "fused_dim", "fused_fp8") else "token"
    fused = mode.startswith("fused")
    if layout == "dim" and fp8:
        vp = vp.view(torch.uint8).transpose(2, 3).contiguous().view(torch.float8_e4m3fn)
    elif layout == "dim":
        vp = vp.transpose(2, 3).contiguous()
    scale = 0.25 if fp8 else 1.0
    sp = 2 if mode in ("split", "fp8_split") else 0
    bits = torch.from_numpy(pack_mask_bits(w.masks).view(np.int64)).cuda()
    tables = torch.empty((w.B, w.Hkv, w.nkvb_max), dtype=torch.int32, device="cuda")
    counts = torch.empty((w.B, w.Hkv), dtype=torch.int32, device="cuda")
    out = torch.empty_like(dv["q"])
    lse = torch.empty((dv["q"].shape[0], w.Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(cpa.split_workspace_bytes(dv["q"].shape[0], w.Hq, w.d, w.nkvb_max, max(sp, 1)), 16),
                     dtype=torch.uint8, device="cuda")

    def step():
        if fused:   # one launch, no tables
            cpa.chunked_prefill_fused(dv["q"], kp, vp, dv["pm"], dv["masks"], dv["cu"], dv["pl"], w.max_chunk_len,
                                      out=out, lse=lse, v_layout=layout, k_scale=scale, v_scale=scale)
            return
        if mode == "bits":
            cpa.build_block_tables_bits(bits, w.nkvb_max, dv["pb"], dv["cb"], w.Hkv, tables=tables, counts=counts)
        else:
            cpa.build_block_tables(dv["masks"], dv["pb"], dv["cb"], w.Hkv, tables=tables, counts=counts)
        cpa.chunked_prefill(dv["q"], kp, vp, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                            out=out, lse=lse, split_pages=sp, workspace=ws if sp else None, v_layout=layout,
                            k_scale=scale, v_scale=scale)

    step()
    torch.cuda.synchronize()
    o_ref, l_ref, t_ref = out.clone(), lse.clone(), tables.clone()
    if fused:   # the same bits as the two separate launches
        tb, cn = cpa.build_block_tables(dv["masks"], dv["pb"], dv["cb"], w.Hkv)
        o_sep, l_sep = cpa.chunked_prefill(dv["q"], kp, vp, dv["pm"], tb, cn, dv["cu"], dv["pl"], w.max_chunk_len,
                                           return_lse=True, v_layout=layout, k_scale=scale, v_scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o_ref, o_sep) and torch.equal(l_ref, l_sep)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm the capture stream, as torch's graph docs ask
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        out.zero_()
        lse.zero_()
        tables.fill_(-7)
        x = torch.randn(1 << 20, device="cuda")   # eager work between the replays
        (x * 2).sum().item()
        g.replay()
        torch.cuda.synchronize()
        if not fused:
            assert torch.equal(tables, t_ref), f"replay {i}: tables"
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), f"replay {i}: output"
