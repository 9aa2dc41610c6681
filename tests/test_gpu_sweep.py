"""Seeded sweep of the whole path over random shapes within the documented limits.

Each case draws a batch (1-4 sequences, prefixes of 0-40 blocks, chunks of 0-400 tokens, so
ragged query tiles, partial last pages and empty chunks occur), a group size (1, 2, 4, 8, 12, 16;
a second draw takes any size 1-16) with 1-3 KV groups, d 64 or 128, a mask density from empty to
full, and one way to run attention: bf16, fp32 or fp8 pools, token- or dim-major V, split-KV or
not.  It then runs the path as a caller would, against the oracle at every step:

  append   the chunk's own K/V rows into the paged pools: bit-exact against the oracle's copy;
  tables   from byte masks and from bit-packed masks: bit-exact;
  attend   over the appended pools: the bars of the hand-picked cases, LSE included;
  direct   (bf16 cases) the per-head baseline's plans bit-exact and its output within the bars;
  fused    (bf16 cases) the table build in the prefill's prologue, bitwise the separate launches.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_reduce_amd as cpa
from workloads import make_workload
from workloads.configs import mask_all, mask_bernoulli, pack_mask_bits

from _gpu import compare, sample_rows, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

N_CASES = int(os.environ.get("CPA_SWEEP_CASES", "32"))   # more for a longer soak of the same draw


def draw(i):
    rng = np.random.default_rng(7000 + i)
    B = int(rng.integers(1, 5))
    chunk = rng.integers(0, 401, size=B)
    if chunk.max() == 0:
        chunk[0] = int(rng.integers(1, 200))
    G = int(rng.choice([1, 2, 4, 8, 12, 16]))
    mode = str(rng.choice(["bf16", "bf16", "f32", "fp8"]))
    c = dict(prefix=(64 * rng.integers(0, 41, size=B)).tolist(), chunk=chunk.tolist(), G=G,
             Hkv=int(rng.integers(1, 3 if G >= 8 else 4)), d=int(rng.choice([64, 128])),
             p=float(rng.choice([-1.0, 0.0, 0.02, 0.1, 0.4, 1.0])), local=int(rng.integers(0, 3)),
             mode=mode, v_layout=str(rng.choice(["token", "dim"])),
             split=int(rng.choice([0, 0, 1, 3, 8])) if mode == "bf16" else 0,
             scales=(float(rng.choice([0.25, 1.0, 3.0])), float(rng.choice([0.5, 2.0]))))
    if mode == "fp8":   # fp8 pools split too; a stream of their own leaves every other draw as it was
        c["split"] = int(np.random.default_rng(7300 + i).choice([0, 0, 1, 3, 8]))
    return c


def mask_fn(c):
    if c["p"] < 0:   # nothing selected at all: empty tables, zero output, LSE -inf
        return lambda rng, *a: mask_all(rng, *a, value=0)
    return lambda rng, *a: mask_bernoulli(rng, *a, p=c["p"], local=c["local"])


def check_lse(lse, L, tol):
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L.T)
    assert np.array_equal(np.isfinite(lg), fin)
    if fin.any():
        assert np.max(np.abs(lg[fin] - L.T[fin])) < tol


def fp8_codes(x, scale):
    return (torch.from_numpy(np.ascontiguousarray(x)) / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep(i):
    c = draw(i)
    print(f"\n[case] sweep {i}: {c}", flush=True)
    run_case(i, c, 7100 + i, 7200 + i)


N_ANY_G = int(os.environ.get("CPA_SWEEP_ANY_G_CASES", "16"))


def draw_any_group(i):
    # the same draw with any group size 1-16 (3, 5, 6, 7, 9, ... included)
    c = draw(i)
    rng = np.random.default_rng(7800 + i)
    c["G"] = int(rng.integers(1, 17))
    c["Hkv"] = int(rng.integers(1, 4))
    return c


@pytest.mark.parametrize("i", range(N_ANY_G))
def test_sweep_any_group(i):
    c = draw_any_group(i)
    print(f"\n[case] any-group sweep {i}: {c}", flush=True)
    run_case(i, c, 7900 + i, 8000 + i)


def run_case(i, c, wseed, rseed):
    Hq, Hkv, d, mode = c["G"] * c["Hkv"], c["Hkv"], c["d"], c["mode"]
    w = make_workload(f"sweep{i}", c["prefix"], c["chunk"], Hq, Hkv, d, "f32" if mode == "f32" else "bf16",
                      mask_fn(c), wseed)
    dv = upload(w)
    rng = np.random.default_rng(rseed)
    new = rng.standard_normal((2, w.q.shape[0], Hkv, d), dtype=np.float32)
    if mode == "fp8":
        ks, vs = c["scales"]
        kpool, vpool = fp8_codes(w.k_pages, ks), fp8_codes(w.v_pages, vs)
        knew, vnew = fp8_codes(new[0], ks), fp8_codes(new[1], vs)
        to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().view(torch.float8_e4m3fn)  # noqa: E731
        back = lambda t: t.view(torch.uint8).cpu().numpy()  # noqa: E731
    else:
        ks = vs = 1.0
        dt = torch.bfloat16 if mode == "bf16" else torch.float32
        kpool, vpool = w.k_pages, w.v_pages
        knew, vnew = [torch.from_numpy(x).to(dt).float().numpy() for x in new]   # representable in dt
        to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)  # noqa: E731
        back = lambda t: t.float().cpu().numpy()  # noqa: E731

    # append: the chunk's rows into their slots, bit for bit as the oracle's copy
    Ko, Vo = oracle.append_kv(knew, vnew, kpool, vpool, w.page_map, w.cu_q, w.prefix_len)
    dim = c["v_layout"] == "dim"
    kp = to_dev(kpool)
    vp = to_dev(np.swapaxes(vpool, 2, 3) if dim else vpool)
    cpa.append_kv(to_dev(knew), to_dev(vnew), kp, vp, dv["pm"], dv["cu"], dv["pl"], w.max_chunk_len,
                  v_layout=c["v_layout"])
    torch.cuda.synchronize()
    assert np.array_equal(back(kp), Ko)
    assert np.array_equal(back(vp), np.swapaxes(Vo, 2, 3) if dim else Vo)

    # tables, from bytes and from bits
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, Hkv, w.nkvb_max)
    tables, counts = cpa.build_block_tables(dv["masks"], dv["pb"], dv["cb"], Hkv)
    assert np.array_equal(tables.cpu().numpy(), T) and np.array_equal(counts.cpu().numpy(), C)
    bits = torch.from_numpy(pack_mask_bits(w.masks).view(np.int64)).cuda()
    tb, cb = cpa.build_block_tables_bits(bits, w.nkvb_max, dv["pb"], dv["cb"], Hkv)
    assert np.array_equal(tb.cpu().numpy(), T) and np.array_equal(cb.cpu().numpy(), C)

    # attention over the appended pools
    if mode == "fp8":
        Kd, Vd = oracle.dequant_e4m3(Ko, ks), oracle.dequant_e4m3(Vo, vs)
    else:
        Kd, Vd = Ko, Vo
    o, lse = cpa.chunked_prefill(dv["q"], kp, vp, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                                 return_lse=True, v_layout=c["v_layout"], split_pages=c["split"],
                                 k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    O, L = oracle.paged_attention(w.q, Kd, Vd, w.page_map, T, C, w.cu_q, w.prefix_len, Hkv)
    compare(w, o, O, f"sweep {i}")
    check_lse(lse, L, 1e-4 if mode == "f32" else (2e-2 if mode == "fp8" else 2 ** -7))
    if c["p"] < 0:
        assert torch.all(o == 0)

    if mode == "fp8":   # the fused launch over the same fp8 pools: bitwise the separate launches
        of, lf = cpa.chunked_prefill_fused(dv["q"], kp, vp, dv["pm"], dv["masks"], dv["cu"], dv["pl"],
                                           w.max_chunk_len, return_lse=True, v_layout=c["v_layout"],
                                           split_pages=c["split"], k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
        assert torch.equal(of.view(torch.int16), o.view(torch.int16)), f"sweep {i} fused fp8 output"
        assert torch.equal(lf.view(torch.int32), lse.view(torch.int32)), f"sweep {i} fused fp8 LSE"

    # the direct baseline on the same pools
    if mode == "bf16":
        plans, pc = cpa.build_block_plans(dv["masks"], dv["pb"], dv["cb"])
        Pn, Cn = oracle.block_plans(w.masks, w.prefix_blocks, w.chunk_blocks, w.nkvb_max)
        assert np.array_equal(plans.cpu().numpy(), Pn) and np.array_equal(pc.cpu().numpy(), Cn)
        vpd = vp if dim else vp.transpose(2, 3).contiguous()
        od, ld = cpa.chunked_prefill_direct(dv["q"], kp, vpd, dv["pm"], plans, pc, dv["cu"], dv["pl"],
                                            w.max_chunk_len, return_lse=True)
        torch.cuda.synchronize()
        Od, Ld = oracle.block_sparse_attention(w.q, Ko, Vo, w.page_map, Pn, Cn, w.cu_q, w.prefix_len, Hkv)
        compare(w, od, Od, f"sweep {i} direct")
        check_lse(ld, Ld, 2 ** -7)

        # the table build in the prefill's prologue: bitwise the separate launches, split or not
        of, lf = cpa.chunked_prefill_fused(dv["q"], kp, vp, dv["pm"], dv["masks"], dv["cu"], dv["pl"],
                                           w.max_chunk_len, return_lse=True, v_layout=c["v_layout"],
                                           split_pages=c["split"])
        ob, lb = cpa.chunked_prefill_fused(dv["q"], kp, vp, dv["pm"], bits, dv["cu"], dv["pl"], w.max_chunk_len,
                                           return_lse=True, v_layout=c["v_layout"], split_pages=c["split"],
                                           nkvb_max=w.nkvb_max)
        torch.cuda.synchronize()
        assert torch.equal(of.view(torch.int16), o.view(torch.int16)), f"sweep {i} fused output"
        assert torch.equal(lf.view(torch.int32), lse.view(torch.int32)), f"sweep {i} fused LSE"
        assert torch.equal(ob.view(torch.int16), o.view(torch.int16)), f"sweep {i} fused output (bit masks)"
        assert torch.equal(lb.view(torch.int32), lse.view(torch.int32)), f"sweep {i} fused LSE (bit masks)"


N_LONG = int(os.environ.get("CPA_SWEEP_LONG_CASES", "12"))


def draw_long(i):
    rng = np.random.default_rng(7500 + i)
    B = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4, 8, 12, 16]))
    mode = str(rng.choice(["bf16", "bf16", "f32"]))
    return dict(prefix=(64 * rng.integers(1000, 1601, size=B)).tolist(), chunk=rng.integers(1, 601, size=B).tolist(),
                G=G, Hkv=int(rng.integers(1, 3)), d=int(rng.choice([64, 128])),
                p=float(rng.choice([0.05, 0.5, 1.0])), local=int(rng.integers(0, 3)), mode=mode,
                v_layout=str(rng.choice(["token", "dim"])),
                split=int(rng.choice([0, 64, 256])) if mode == "bf16" else 0)


@pytest.mark.parametrize("i", range(N_LONG))
def test_sweep_long(i):
    # contexts of 64K-102K tokens: tables of hundreds to 1600 pages, most past the kernel's window
    # of 1024 resolved page ids; tables in full, attention on sampled rows
    c = draw_long(i)
    print(f"\n[case] long sweep {i}: {c}", flush=True)
    Hq, Hkv = c["G"] * c["Hkv"], c["Hkv"]
    w = make_workload(f"long{i}", c["prefix"], c["chunk"], Hq, Hkv, c["d"], c["mode"], mask_fn(c), 7600 + i)
    dv = upload(w)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, Hkv, w.nkvb_max)
    tables, counts = cpa.build_block_tables(dv["masks"], dv["pb"], dv["cb"], Hkv)
    assert np.array_equal(tables.cpu().numpy(), T) and np.array_equal(counts.cpu().numpy(), C)
    vp = dv["vp"].transpose(2, 3).contiguous() if c["v_layout"] == "dim" else dv["vp"]
    o, lse = cpa.chunked_prefill(dv["q"], dv["kp"], vp, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                                 return_lse=True, v_layout=c["v_layout"], split_pages=c["split"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    S = sample_rows(w, 96, seed=i)
    Os, Ls = oracle.attention_rows(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, Hkv, S)
    r = torch.from_numpy(w.cu_q[S[:, 0]] + S[:, 2]).cuda()
    h = torch.from_numpy(S[:, 1]).cuda()
    compare(w, o[r, h].float().cpu().numpy(), Os, f"long sweep {i}")
    assert np.max(np.abs(lse[r, h].cpu().numpy() - Ls)) < (1e-4 if c["mode"] == "f32" else 2 ** -7)
    if c["mode"] == "bf16":   # the fused launch expands these long tables from its bitmap, window by window
        of, lf = cpa.chunked_prefill_fused(dv["q"], dv["kp"], vp, dv["pm"], dv["masks"], dv["cu"], dv["pl"],
                                           w.max_chunk_len, return_lse=True, v_layout=c["v_layout"],
                                           split_pages=c["split"])
        torch.cuda.synchronize()
        assert torch.equal(of.view(torch.int16), o.view(torch.int16)), f"long sweep {i} fused output"
        assert torch.equal(lf.view(torch.int32), lse.view(torch.int32)), f"long sweep {i} fused LSE"
