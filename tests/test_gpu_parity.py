"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tables must match bit for bit (whole buffers, -1 tail included).  Outputs must be within
max-abs 1e-4 of the oracle for fp32 inputs, and within max-abs 2e-2 and mean-abs 2e-3 for bf16
inputs.  Small cases compare every output element; the full-size workloads, run through the
same entry points the benchmark times, compare sampled rows that the oracle computes one by one
and check size-independent properties on every row.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import make_config, make_workload
from workloads.configs import mask_all, mask_bernoulli, mask_stripes, mask_structured

import sparse_attention_long_reduce_amd as cpa

from _gpu import compare, error_stats, gpu_prefill, gpu_tables, oracle_full, report, sample_rows, tiles_reached, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def oracle_tables(w, cap=None):
    return oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv,
                                     w.nkvb_max if cap is None else cap)


def oracle_out(w, T, C):
    return oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q,
                                  w.prefix_len, w.Hkv)


def bern(p, local=1):
    return lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=local)


# small variants: (name, kwargs for make_workload)
SMALL = {
    "tiny_sparse_g4_bf16": dict(prefix_len=[768], chunk_len=[256], Hq=8, Hkv=2, d=64, dtype="bf16", mask_fn=bern(0.05)),
    "tiny_sparse_g1_f32": dict(prefix_len=[768], chunk_len=[256], Hq=2, Hkv=2, d=64, dtype="f32", mask_fn=bern(0.05)),
    "g2_varlen_bf16_d128": dict(prefix_len=[0, 640, 1280], chunk_len=[320, 192, 64], Hq=4, Hkv=2, d=128, dtype="bf16", mask_fn=bern(0.1)),
    "g8_bf16_d128": dict(prefix_len=[512], chunk_len=[256], Hq=16, Hkv=2, d=128, dtype="bf16", mask_fn=bern(0.1)),
    "g1_f32_d128_ragged": dict(prefix_len=[320, 0], chunk_len=[100, 77], Hq=3, Hkv=3, d=128, dtype="f32", mask_fn=bern(0.2)),
    "g4_bf16_ragged_multi": dict(prefix_len=[0, 192, 4096], chunk_len=[37, 130, 255], Hq=8, Hkv=2, d=128, dtype="bf16", mask_fn=bern(0.05)),
    "g4_f32_d64_noise": dict(prefix_len=[448, 64], chunk_len=[192, 256], Hq=8, Hkv=2, d=64, dtype="f32", mask_fn=bern(0.1), noncausal_noise=0.3, mask_values=True),
    "partial_word_70": dict(prefix_len=[64 * 66], chunk_len=[256], Hq=8, Hkv=2, d=64, dtype="bf16", mask_fn=bern(0.03)),
    "nqb1": dict(prefix_len=[1024], chunk_len=[64], Hq=8, Hkv=2, d=128, dtype="bf16", mask_fn=bern(0.2)),
    "all_ones_f32": dict(prefix_len=[256, 0], chunk_len=[192, 128], Hq=8, Hkv=2, d=64, dtype="f32", mask_fn=lambda rng, *a: mask_all(rng, *a, value=1)),
    "all_zero_bf16": dict(prefix_len=[256], chunk_len=[128], Hq=8, Hkv=2, d=128, dtype="bf16", mask_fn=lambda rng, *a: mask_all(rng, *a, value=0)),
    "stripes_g4_f32_d128": dict(prefix_len=[1536], chunk_len=[512], Hq=8, Hkv=2, d=128, dtype="f32", mask_fn=lambda rng, *a: mask_stripes(rng, *a, p=0.1, shared_per_group=False)),
    "zero_len_chunk": dict(prefix_len=[128, 256], chunk_len=[0, 128], Hq=8, Hkv=2, d=64, dtype="bf16", mask_fn=bern(0.3)),
    # group sizes that are not powers of two: a workgroup's four (query block, head) pairs then
    # span two query blocks, and tiles end inside a query block's heads
    "g3_bf16_ragged": dict(prefix_len=[0, 448], chunk_len=[200, 129], Hq=6, Hkv=2, d=128, dtype="bf16", mask_fn=bern(0.1)),
    "g5_bf16_d64": dict(prefix_len=[320], chunk_len=[250], Hq=5, Hkv=1, d=64, dtype="bf16", mask_fn=bern(0.15)),
    "g6_f32_d64": dict(prefix_len=[256, 0], chunk_len=[192, 70], Hq=12, Hkv=2, d=64, dtype="f32", mask_fn=bern(0.2)),
    "g7_bf16_d128": dict(prefix_len=[640, 64], chunk_len=[300, 64], Hq=14, Hkv=2, d=128, dtype="bf16", mask_fn=bern(0.1)),
    "g7_f32_d128": dict(prefix_len=[128], chunk_len=[190], Hq=7, Hkv=1, d=128, dtype="f32", mask_fn=bern(0.3)),
    "g12_bf16_d64": dict(prefix_len=[192, 512], chunk_len=[128, 65], Hq=24, Hkv=2, d=64, dtype="bf16", mask_fn=bern(0.1)),
}


def make_small(name, seed=11):
    kw = dict(SMALL[name])
    return make_workload(name, kw.pop("prefix_len"), kw.pop("chunk_len"), kw.pop("Hq"), kw.pop("Hkv"),
                         kw.pop("d"), kw.pop("dtype"), kw.pop("mask_fn"), seed, **kw)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_tables_and_prefill(name):
    print(f"\n[case] small {name}", flush=True)
    w = make_small(name)
    dv = upload(w)
    cap = w.nkvb_max + 5
    tables, counts = gpu_tables(dv, w, cap)
    T, C = oracle_tables(w, cap)
    assert np.array_equal(tables.cpu().numpy(), T)
    assert np.array_equal(counts.cpu().numpy(), C)
    o, lse = gpu_prefill(dv, w, tables, counts)
    torch.cuda.synchronize()
    O, L = oracle_out(w, T, C)
    compare(w, o, O, name)
    lg = lse.cpu().numpy().astype(np.float64)
    Lr = L.T
    fin = np.isfinite(Lr)
    assert np.array_equal(np.isfinite(lg), fin)
    if fin.any():
        # bf16 path: the row sum adds the bf16-rounded weights (relative rounding <= 2^-9 each,
        # <= 2^-9 on the LSE), and Q is rounded to bf16 after the softmax scale is folded in,
        # which moves a score by 2^-9/sqrt(3) * scale * |q.k|_2 ~ 1.1e-3 RMS at d = 128 with
        # N(0,1) inputs; a row dominated by one key carries that into the LSE (5 sigma 5.7e-3)
        tol = 2 ** -7 if w.dtype == "bf16" else 1e-4
        assert np.max(np.abs(lg[fin] - Lr[fin])) < tol
    if name == "all_zero_bf16":
        assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("cap_extra", [0, 1, 7])
def test_tables_one_block_sequences(cap_extra):
    # one KV block per sequence, at the minimum capacity and above it
    w = make_workload("one_block", [0, 0, 0], [40, 64, 1], 8, 2, 64, "bf16", bern(0.5), 6)
    assert w.nkvb_max == 1
    dv = upload(w)
    cap = 1 + cap_extra
    tables, counts = gpu_tables(dv, w, cap)
    T, C = oracle_tables(w, cap)
    assert np.array_equal(tables.cpu().numpy(), T) and np.array_equal(counts.cpu().numpy(), C)


@pytest.mark.parametrize("nkvb", [3, 63, 64, 65, 129])
def test_tables_word_boundaries(nkvb):
    # extents around the 64-block words of the build's bitsets and 16-block load columns, at the
    # minimum capacity, from bytes and from bit-packed masks
    w = make_workload(f"w{nkvb}", [64 * (nkvb - 2)], [128], 8, 2, 64, "bf16", bern(0.3), nkvb,
                      noncausal_noise=0.2)
    assert w.nkvb_max == nkvb
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle_tables(w)
    assert np.array_equal(tables.cpu().numpy(), T) and np.array_equal(counts.cpu().numpy(), C)
    from workloads.configs import pack_mask_bits
    bits = torch.from_numpy(pack_mask_bits(w.masks).view(np.int64)).cuda()
    t2, c2 = cpa.build_block_tables_bits(bits, w.nkvb_max, dv["pb"], dv["cb"], w.Hkv)
    assert np.array_equal(t2.cpu().numpy(), T) and np.array_equal(c2.cpu().numpy(), C)


def test_tables_unaligned_mask_width():
    # nkvb_max = 70 is not a multiple of 16: the byte path of the union kernel
    w = make_workload("w70", [64 * 66], [256], 8, 2, 64, "bf16", bern(0.03), 5, noncausal_noise=0.2)
    assert w.nkvb_max == 70
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle_tables(w)
    assert np.array_equal(tables.cpu().numpy(), T) and np.array_equal(counts.cpu().numpy(), C)


_CACHE = {}


def config(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _CACHE:
        _CACHE.clear()
        _CACHE[key] = make_config(name, **kw)
    return _CACHE[key]


def test_config1_full():
    print("\n[case] c1_tiny_f32 full", flush=True)
    w = config("c1_tiny_f32")
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle_tables(w)
    assert np.array_equal(tables.cpu().numpy(), T) and np.array_equal(counts.cpu().numpy(), C)
    o, lse = gpu_prefill(dv, w, tables, counts)
    O, L = oracle_out(w, T, C)
    compare(w, o, O, "c1")
    assert np.max(np.abs(lse.cpu().numpy() - L.T)) < 1e-4


BIG = [("c2_32k_bf16", {}), ("c3_128k_last_chunk", {}), ("c4_128k_chunked", {"chunk": 0}),
       ("c4_128k_chunked", {"chunk": 17}), ("c4_128k_chunked", {"chunk": 63}),
       ("c5a_varlen_shared", {}), ("c5b_varlen_independent", {}), ("c3_128k_last_chunk", {"dense": True}),
       ("c3d_128k_no_noise", {}), ("c3g7_128k_gqa7", {})]


@pytest.mark.parametrize("name,kw", BIG, ids=[f"{n}{kw}" for n, kw in BIG])
def test_full_size_configs(name, kw):
    print(f"\n[case] {name} {kw}", flush=True)
    w = config(name, **kw)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle_tables(w)
    assert np.array_equal(tables.cpu().numpy(), T), "tables differ"
    assert np.array_equal(counts.cpu().numpy(), C), "counts differ"
    o, lse = gpu_prefill(dv, w, tables, counts)
    torch.cuda.synchronize()
    # properties on every row: finite, convex combination of V rows
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    vmax = float(dv["vp"].abs().max())
    assert float(o.abs().max()) <= vmax * (1 + 2 ** -7)
    # sampled rows against the oracle: 384 random rows plus two rows of every (sequence, KV
    # group, query block) tile, one in each 32-row half
    S = sample_rows(w, 384, seed=1)
    reached, total = tiles_reached(w, S)
    assert reached == total
    Os, Ls = oracle.attention_rows(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len,
                                   w.Hkv, S)
    rows = torch.from_numpy(w.cu_q[S[:, 0]] + S[:, 2]).cuda()
    heads = torch.from_numpy(S[:, 1]).cuda()
    og = o[rows, heads].float().cpu().numpy()
    compare(w, og, Os, f"{name}{kw}")
    report(f"sampled {name}{kw} ({len(S)} rows, {total} tiles)", error_stats(og, Os))
    lg = lse[rows, heads].cpu().numpy()
    assert np.max(np.abs(lg - Ls)) < 2e-2


WHOLE = ["c2_32k_bf16", "c3_128k_last_chunk", "c5a_varlen_shared", "c5b_varlen_independent"]


@pytest.mark.parametrize("name", WHOLE)
def test_whole_output_against_oracle(name):
    # every output element of the workload, in the layout the benchmark times (dim-major V),
    # against the oracle; the tolerances are the bf16 bars, and the errors are reported
    print(f"\n[case] whole output {name}", flush=True)
    w = config(name)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle_tables(w)
    assert np.array_equal(tables.cpu().numpy(), T) and np.array_equal(counts.cpu().numpy(), C)
    vdim = dv["vp"].transpose(2, 3).contiguous()
    o, lse = cpa.chunked_prefill(dv["q"], dv["kp"], vdim, dv["pm"], tables, counts, dv["cu"], dv["pl"],
                                 w.max_chunk_len, return_lse=True, v_layout="dim")
    torch.cuda.synchronize()
    O, L = oracle_full(w, T, C)
    compare(w, o, O, f"whole {name}")
    st = error_stats(o, O)
    lg = lse.cpu().numpy().astype(np.float64)
    st["lse_max_abs"] = float(np.max(np.abs(lg - L.T)))
    report(f"whole {name}", st)
    assert st["lse_max_abs"] < 2 ** -7


def poisoned(w, T, C, value=np.nan):
    """Copies of the pools with every page no table entry reaches set to `value`."""
    keep = np.zeros(w.n_pages, dtype=bool)
    for b in range(w.B):
        for g in range(w.Hkv):
            keep[w.page_map[b, T[b, g, :C[b, g]]]] = True
    kp = w.k_pages.copy()
    vp = w.v_pages.copy()
    kp[~keep] = value
    vp[~keep] = value
    return kp, vp, int((~keep).sum())


@pytest.mark.parametrize("name", ["tiny_sparse_g4_bf16", "g4_bf16_ragged_multi", "stripes_g4_f32_d128"])
def test_poison_unselected_pages(name):
    w = make_small(name)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle_tables(w)
    o1, l1 = gpu_prefill(dv, w, tables, counts)
    kp, vp, n = poisoned(w, T, C)
    assert n > 0
    dt = dv["q"].dtype
    o2, l2 = gpu_prefill(dv, w, tables, counts, kp=torch.from_numpy(kp).cuda().to(dt),
                         vp=torch.from_numpy(vp).cuda().to(dt))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_poison_unselected_pages_128k():
    w = config("c3_128k_last_chunk")
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle_tables(w)
    o1, l1 = gpu_prefill(dv, w, tables, counts)
    kp, vp, n = poisoned(w, T, C)
    assert n > 500
    o2, l2 = gpu_prefill(dv, w, tables, counts, kp=torch.from_numpy(kp).cuda().to(torch.bfloat16),
                         vp=torch.from_numpy(vp).cuda().to(torch.bfloat16))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_attribution(dtype):
    # V one-hot by block: output channel kb % d carries block kb's softmax mass, so a missed or
    # extra block shifts a channel by far more than the tolerance
    w = make_workload("attr", [64 * 60], [256], 8, 2, 128, dtype,
                      lambda rng, *a: mask_stripes(rng, *a, p=0.3, shared_per_group=False), 21)
    for b in range(w.B):
        for kb in range(w.page_map.shape[1]):
            pg = w.page_map[b, kb]
            w.v_pages[pg] = 0
            w.v_pages[pg, :, :, kb % w.d] = 1
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle_tables(w)
    o, _ = gpu_prefill(dv, w, tables, counts)
    O, _ = oracle_out(w, T, C)
    compare(w, o, O, "attribution")
    on = o.float().cpu().numpy()
    # channels of blocks outside the table are exactly zero
    for h in range(w.Hq):
        g = h // w.G
        sel = {int(k) % w.d for k in T[0, g, :C[0, g]]}
        unsel = [c for c in range(w.d) if c not in sel]
        assert np.all(on[:, h, unsel] == 0)


def test_determinism_and_page_permutation():
    w = make_small("g4_bf16_ragged_multi")
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    o1, l1 = gpu_prefill(dv, w, tables, counts)
    o2, l2 = gpu_prefill(dv, w, tables, counts)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    rng = np.random.default_rng(3)
    perm = rng.permutation(w.n_pages)
    k2 = np.empty_like(w.k_pages)
    v2 = np.empty_like(w.v_pages)
    k2[perm] = w.k_pages
    v2[perm] = w.v_pages
    dv2 = upload(w, k_pages=k2, v_pages=v2, page_map=perm[w.page_map].astype(np.int32))
    o3, l3 = gpu_prefill(dv2, w, tables, counts)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_strided_kv_pool():
    # K and V interleaved in one pool [n_pages][2][Hkv][64][d]; the kernel gets strided views
    w = make_small("g2_varlen_bf16_d128")
    dv = upload(w)
    pool = torch.stack([dv["kp"], dv["vp"]], dim=1).contiguous()
    tables, counts = gpu_tables(dv, w)
    o1, l1 = gpu_prefill(dv, w, tables, counts)
    o2, l2 = gpu_prefill(dv, w, tables, counts, kp=pool[:, 0], vp=pool[:, 1])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_out_of_range_page_ids_read_as_nan():
    w = make_small("tiny_sparse_g4_bf16")
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle_tables(w)
    only1 = sorted(set(T[0, 1, :C[0, 1]].tolist()) - set(T[0, 0, :C[0, 0]].tolist()))
    assert only1, "need a block selected by group 1 only"
    kb = only1[0]
    pm = w.page_map.copy()
    pm[0, kb] = w.n_pages + 5              # that block's page id now points outside the pool
    dv["pm"] = torch.from_numpy(pm).cuda()
    o, lse = gpu_prefill(dv, w, tables, counts)
    on = o.float().cpu().numpy()
    rows_seeing = np.arange(int(w.chunk_len[0])) + int(w.prefix_len[0]) >= 64 * kb
    assert np.all(np.isnan(on[rows_seeing][:, 4:8]))      # group 1's heads on rows that reach kb
    assert not np.any(np.isnan(on[~rows_seeing][:, 4:8]))
    O, _ = oracle_out(w, T, C)
    compare(w, o[:, :4], O[:, :4], "group 0 unaffected")


def test_sm_scale_argument():
    w = make_small("g4_f32_d64_noise")
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle_tables(w)
    import sparse_attention_long_reduce_amd as cpa
    o, _ = cpa.chunked_prefill(dv["q"], dv["kp"], dv["vp"], dv["pm"], tables, counts, dv["cu"],
                               dv["pl"], w.max_chunk_len, sm_scale=0.05)
    O, _ = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len,
                                  w.Hkv, scale=0.05)
    compare(w, o, O, "sm_scale")


@pytest.mark.parametrize("name", ["c3_128k_last_chunk", "c5b_varlen_independent"])
def test_prescaled_q_rounding_cost(name):
    # The bf16 kernel multiplies Q by scale * log2(e) and rounds the product back to bf16 before
    # the QK product (an input rounding the plain definition does not have).  Its cost: the error
    # of the GPU against the oracle on the original Q, against the oracle on that rounded Q (what
    # the kernel's products see), and between the two oracles, on rows reaching every tile.
    from workloads.configs import bf16_round
    print(f"\n[case] pre-scaled Q rounding {name}", flush=True)
    w = config(name)
    dv = upload(w)
    tables, counts = gpu_tables(dv, w)
    T, C = oracle_tables(w)
    o, lse = gpu_prefill(dv, w, tables, counts)
    torch.cuda.synchronize()
    S = sample_rows(w, 384, seed=4)
    cs32 = np.float32(np.float32(1.0) / np.sqrt(np.float32(w.d))) * np.float32(1.4426950408889634)
    q_r = bf16_round(w.q.astype(np.float32) * cs32).astype(np.float64) / (math.log2(math.e) / math.sqrt(w.d))
    O, _ = oracle.attention_rows(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv, S)
    O_r, _ = oracle.attention_rows(q_r, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv, S)
    rows = torch.from_numpy(w.cu_q[S[:, 0]] + S[:, 2]).cuda()
    og = o[rows, torch.from_numpy(S[:, 1]).cuda()].float().cpu().numpy()
    e_def, e_rnd, e_ora = error_stats(og, O), error_stats(og, O_r), error_stats(O_r, O)
    report(f"q-rounding {name}: gpu vs oracle(q)", e_def)
    report(f"q-rounding {name}: gpu vs oracle(rounded q)", e_rnd)
    report(f"q-rounding {name}: oracle(rounded q) vs oracle(q)", e_ora)
    compare(w, og, O, name)
    # the rounding of Q is a small part of the bf16 budget: the oracles differ far below the bars
    assert e_ora["max_abs"] < 2e-3 and e_ora["mean_abs"] < 2e-4
