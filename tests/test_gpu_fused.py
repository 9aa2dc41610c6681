"""GPU parity of the fused entry point (cpa_chunked_prefill_fused: the block union built in the
prefill's prologue, one launch) against the fp64 CPU oracle, and against the separate
table-build + prefill launches, which it must reproduce bit for bit: it visits the same pages
in the same order, so every floating-point operation is the same."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_reduce_amd as cpa
from workloads import make_config, make_workload
from workloads.configs import chunked_sequence_batch, mask_all, mask_bernoulli, pack_mask_bits

from _gpu import compare, error_stats, report, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def bern(p, local=1):
    return lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=local)


SMALL = {
    "g4_bf16_d128": dict(prefix_len=[1024], chunk_len=[256], Hq=8, Hkv=2, d=128, mask_fn=bern(0.05)),
    "g4_bf16_d64_noise": dict(prefix_len=[448, 64], chunk_len=[192, 256], Hq=8, Hkv=2, d=64, mask_fn=bern(0.1),
                              noncausal_noise=0.3, mask_values=True),
    "g1_bf16_ragged": dict(prefix_len=[1024, 64], chunk_len=[192, 100], Hq=2, Hkv=2, d=128, mask_fn=bern(0.3)),
    "g2_varlen_d128": dict(prefix_len=[0, 640, 1280], chunk_len=[320, 192, 64], Hq=4, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g3_bf16_ragged": dict(prefix_len=[0, 448], chunk_len=[200, 129], Hq=6, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g5_bf16_d64": dict(prefix_len=[320], chunk_len=[250], Hq=10, Hkv=2, d=64, mask_fn=bern(0.15)),
    "g7_bf16_d128": dict(prefix_len=[640, 64], chunk_len=[300, 64], Hq=14, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g8_bf16_d128": dict(prefix_len=[512], chunk_len=[256], Hq=16, Hkv=2, d=128, mask_fn=bern(0.1)),
    "g4_ragged_multi_8groups": dict(prefix_len=[0, 192, 4096, 320], chunk_len=[37, 130, 255, 64], Hq=8, Hkv=2, d=128,
                                    mask_fn=bern(0.05)),
    "all_zero": dict(prefix_len=[256], chunk_len=[128], Hq=8, Hkv=2, d=128,
                     mask_fn=lambda rng, *a: mask_all(rng, *a, value=0)),
    "zero_len_chunk": dict(prefix_len=[128, 256], chunk_len=[0, 128], Hq=8, Hkv=2, d=64, mask_fn=bern(0.3)),
    # a table longer than one window chunk (512 ids): the ids are expanded from the bitmap in
    # several refills; 2400 blocks also span many 64-bit words
    "long_table_refills": dict(prefix_len=[64 * 2340], chunk_len=[64], Hq=4, Hkv=1, d=64, mask_fn=bern(0.5)),
}


def make_small(name, seed=41):
    kw = dict(SMALL[name])
    return make_workload(name, kw.pop("prefix_len"), kw.pop("chunk_len"), kw.pop("Hq"), kw.pop("Hkv"),
                         kw.pop("d"), "bf16", kw.pop("mask_fn"), seed, **kw)


def dim_major(vp):
    return vp.transpose(2, 3).contiguous()


def fused(dv, w, layout, masks=None, vp=None, split=0):
    if vp is None:
        vp = dim_major(dv["vp"]) if layout == "dim" else dv["vp"]
    return cpa.chunked_prefill_fused(dv["q"], dv["kp"], vp, dv["pm"], dv["masks"] if masks is None else masks,
                                     dv["cu"], dv["pl"], w.max_chunk_len, return_lse=True, v_layout=layout,
                                     split_pages=split)


def fused_bits(dv, w, layout, split=0):
    """The fused launch from the bit-packed form of the workload's masks."""
    vp = dim_major(dv["vp"]) if layout == "dim" else dv["vp"]
    bits = torch.from_numpy(pack_mask_bits(w.masks).view(np.int64)).cuda()
    return cpa.chunked_prefill_fused(dv["q"], dv["kp"], vp, dv["pm"], bits, dv["cu"], dv["pl"], w.max_chunk_len,
                                     return_lse=True, v_layout=layout, split_pages=split, nkvb_max=w.nkvb_max)


def separate(dv, w, layout, masks=None, vp=None, split=0):
    """The table-build launch, then the prefill launch on its tables (capacity: the masks' width)."""
    if vp is None:
        vp = dim_major(dv["vp"]) if layout == "dim" else dv["vp"]
    m = dv["masks"] if masks is None else masks
    tables, counts = cpa.build_block_tables(m, dv["pb"], dv["cb"], w.Hkv, table_cap=max(m.shape[3], 1))
    return cpa.chunked_prefill(dv["q"], dv["kp"], vp, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                               return_lse=True, v_layout=layout, split_pages=split)


def assert_bitwise(a, b, what):
    (o1, l1), (o2, l2) = a, b
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"{what}: outputs differ"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), f"{what}: LSEs differ"


@pytest.mark.parametrize("split", [0, 3])
@pytest.mark.parametrize("layout", ["dim", "token"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_fused_small(name, layout, split):
    w = make_small(name)
    print(f"\n[case] fused {name} v_layout={layout} split_pages={split}", flush=True)
    dv = upload(w)
    got = fused(dv, w, layout, split=split)
    ref = separate(dv, w, layout, split=split)
    torch.cuda.synchronize()
    assert_bitwise(got, ref, name)
    assert_bitwise(fused_bits(dv, w, layout, split=split), ref, f"{name} from bit-packed masks")
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    O, L = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    o, lse = got
    compare(w, o, O, f"{name} fused")
    fin = np.isfinite(L.T)
    lg = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isfinite(lg), fin)
    if fin.any():
        assert np.max(np.abs(lg[fin] - L.T[fin])) < 2 ** -7


KS, VS = 0.37, 1.9   # fp8 dequantization scales


def fp8_pools(w, layout):
    """e4m3 copies of the workload's pools (values / scale), V in the given layout, and the
    oracle's dequantization of the same codes."""
    f8 = torch.float8_e4m3fn
    kc = (torch.from_numpy(w.k_pages) / KS).to(f8)
    vc = (torch.from_numpy(w.v_pages) / VS).to(f8)
    kdq = oracle.dequant_e4m3(kc.view(torch.uint8).numpy(), KS)
    vdq = oracle.dequant_e4m3(vc.view(torch.uint8).numpy(), VS)
    kp, vp = kc.cuda(), vc.cuda()
    if layout == "dim":
        vp = vp.view(torch.uint8).transpose(2, 3).contiguous().view(f8)
    return kp, vp, kdq, vdq


@pytest.mark.parametrize("split", [0, 3])
@pytest.mark.parametrize("layout", ["dim", "token"])
@pytest.mark.parametrize("name", ["g4_bf16_d128", "g2_varlen_d128", "g3_bf16_ragged", "g5_bf16_d64",
                                  "g4_ragged_multi_8groups", "all_zero", "zero_len_chunk", "long_table_refills"])
def test_fused_fp8_small(name, layout, split):
    # fp8 pages: the fused launch reproduces the table build followed by the fp8 prefill (split or
    # not) bit for bit, from byte and from bit-packed masks
    w = make_small(name)
    print(f"\n[case] fused fp8 {name} v_layout={layout} split_pages={split}", flush=True)
    dv = upload(w)
    kp, vp, kdq, vdq = fp8_pools(w, layout)
    got = cpa.chunked_prefill_fused(dv["q"], kp, vp, dv["pm"], dv["masks"], dv["cu"], dv["pl"], w.max_chunk_len,
                                    return_lse=True, v_layout=layout, split_pages=split, k_scale=KS, v_scale=VS)
    bits = torch.from_numpy(pack_mask_bits(w.masks).view(np.int64)).cuda()
    got_bits = cpa.chunked_prefill_fused(dv["q"], kp, vp, dv["pm"], bits, dv["cu"], dv["pl"], w.max_chunk_len,
                                         return_lse=True, v_layout=layout, split_pages=split, nkvb_max=w.nkvb_max,
                                         k_scale=KS, v_scale=VS)
    tables, counts = cpa.build_block_tables(dv["masks"], dv["pb"], dv["cb"], w.Hkv, table_cap=max(w.nkvb_max, 1))
    ref = cpa.chunked_prefill(dv["q"], kp, vp, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                              return_lse=True, v_layout=layout, split_pages=split, k_scale=KS, v_scale=VS)
    torch.cuda.synchronize()
    assert_bitwise(got, ref, f"fp8 {name}")
    assert_bitwise(got_bits, ref, f"fp8 {name} from bit-packed masks")
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    O, L = oracle.paged_attention(w.q, kdq, vdq, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv)
    compare(w, got[0], O, f"fp8 {name} fused")


def test_fused_fp8_full_size_128k():
    # the 128K last chunk over fp8 pages (dim-major V), fused against the separate launches
    print("\n[case] fused fp8 c3 dim", flush=True)
    w = make_config("c3_128k_last_chunk")
    dv = upload(w)
    kp, vp, _, _ = fp8_pools(w, "dim")
    got = cpa.chunked_prefill_fused(dv["q"], kp, vp, dv["pm"], dv["masks"], dv["cu"], dv["pl"], w.max_chunk_len,
                                    return_lse=True, v_layout="dim", k_scale=KS, v_scale=VS)
    tables, counts = cpa.build_block_tables(dv["masks"], dv["pb"], dv["cb"], w.Hkv)
    ref = cpa.chunked_prefill(dv["q"], kp, vp, dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                              return_lse=True, v_layout="dim", k_scale=KS, v_scale=VS)
    torch.cuda.synchronize()
    assert_bitwise(got, ref, "fp8 c3")


def test_fused_unaligned_and_odd_width_masks():
    # masks whose rows are not a multiple of 16 bytes, and masks at an odd address, take the
    # byte-at-a-time reads; padding columns past each sequence's extent hold noise that the
    # clip must drop
    w = make_small("g4_bf16_d64_noise")
    dv = upload(w)
    B, Hq, nqb, nkvb = w.masks.shape
    wide = np.zeros((B, Hq, nqb, nkvb + 3), dtype=np.uint8)
    wide[..., :nkvb] = w.masks
    wide[..., nkvb:] = 7
    m_wide = torch.from_numpy(wide).cuda()
    buf = torch.zeros(w.masks.size + 16, dtype=torch.uint8, device="cuda")
    m_odd = buf[1:1 + w.masks.size].view(w.masks.shape)
    m_odd.copy_(dv["masks"])
    assert m_odd.data_ptr() % 16 == 1 and m_odd.is_contiguous()
    base = fused(dv, w, "dim")
    for m, what in ((m_wide, "width nkvb+3"), (m_odd, "odd base address")):
        for layout in ("dim", "token"):
            assert_bitwise(fused(dv, w, layout, masks=m), separate(dv, w, layout, masks=m), what)
    assert_bitwise(fused(dv, w, "dim", masks=m_wide), base, "padding columns are outside every sequence")
    assert_bitwise(fused(dv, w, "dim", masks=m_odd), base, "same bytes at another address")


def test_fused_masks_narrower_than_the_context():
    # fewer mask rows than query blocks and fewer columns than KV blocks: the union clamps its
    # lengths as the table build does, and both paths agree bit for bit
    w = make_small("g2_varlen_d128")
    dv = upload(w)
    for sl in ((slice(None), slice(None), slice(0, 3), slice(None)),
               (slice(None), slice(None), slice(None), slice(0, 15))):
        m = dv["masks"][sl].contiguous()
        for layout in ("dim", "token"):
            assert_bitwise(fused(dv, w, layout, masks=m), separate(dv, w, layout, masks=m), f"masks {tuple(m.shape)}")


def test_fused_mask_values_do_not_matter():
    # any nonzero byte selects a block
    w = make_small("g3_bf16_ragged")
    dv = upload(w)
    rng = np.random.default_rng(3)
    vals = np.where(w.masks != 0, rng.integers(1, 256, size=w.masks.shape), 0).astype(np.uint8)
    m = torch.from_numpy(vals).cuda()
    assert_bitwise(fused(dv, w, "dim", masks=m), fused(dv, w, "dim"), "byte values")


def test_fused_bits_wider_rows_and_validation():
    # rows of more words than the blocks need (the extra bits are noise the clip drops), and the
    # binding's refusal of bit-packed masks without their block count
    w = make_small("g4_bf16_d64_noise")
    dv = upload(w)
    packed = pack_mask_bits(w.masks).view(np.int64)
    wide = np.full(packed.shape[:-1] + (packed.shape[-1] + 2,), -1, dtype=np.int64)
    wide[..., :packed.shape[-1]] = packed
    last = w.nkvb_max % 64
    if last:   # noise past nkvb_max in the last real word
        wide[..., packed.shape[-1] - 1] |= np.int64(-1) << np.int64(last)
    m = torch.from_numpy(wide).cuda()
    for layout in ("dim", "token"):
        vp = dim_major(dv["vp"]) if layout == "dim" else dv["vp"]
        got = cpa.chunked_prefill_fused(dv["q"], dv["kp"], vp, dv["pm"], m, dv["cu"], dv["pl"], w.max_chunk_len,
                                        return_lse=True, v_layout=layout, nkvb_max=w.nkvb_max)
        assert_bitwise(got, separate(dv, w, layout), f"wide bit rows {layout}")
    with pytest.raises(ValueError, match="nkvb_max"):
        cpa.chunked_prefill_fused(dv["q"], dv["kp"], dv["vp"], dv["pm"], m, dv["cu"], dv["pl"], w.max_chunk_len)


def test_fused_nothing_to_do():
    w = make_small("g4_bf16_d128")
    dv = upload(w)
    o, lse = cpa.chunked_prefill_fused(dv["q"], dv["kp"], dv["vp"], dv["pm"], dv["masks"], dv["cu"], dv["pl"], 0,
                                       return_lse=True)
    torch.cuda.synchronize()   # max_chunk_len 0: no launch, the buffers stay as allocated


@pytest.mark.parametrize("name,layout", [("c3_128k_last_chunk", "dim"), ("c3_128k_last_chunk", "token"),
                                         ("c5b_varlen_independent", "dim"), ("c3g7_128k_gqa7", "dim"),
                                         ("c4_128k_chunked_batch", "dim"), ("c3s_128k_one_group", "dim"),
                                         ("c3s_128k_one_group", "token")])
def test_fused_full_size(name, layout):
    print(f"\n[case] fused full {name} v_layout={layout}", flush=True)
    w = chunked_sequence_batch() if name == "c4_128k_chunked_batch" else make_config(name)
    dv = upload(w)
    sp = 0
    if name.startswith("c3s"):   # one KV group: split-KV, as the bench runs it
        n_cus = torch.cuda.get_device_properties(0).multi_processor_count
        sp = cpa.plan_split_pages(w.B, w.Hq, w.Hkv, w.max_chunk_len, w.nkvb_max, n_cus)
        assert sp > 0
    got = fused(dv, w, layout, split=sp)
    ref = separate(dv, w, layout, split=sp)
    torch.cuda.synchronize()
    assert_bitwise(got, ref, name)
    assert_bitwise(fused_bits(dv, w, layout, split=sp), ref, f"{name} from bit-packed masks")
    o, lse = got
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    # every tile is checked through the bitwise equality with the separate launches, whose own
    # full-size tests reach every tile; a random sample is compared with the oracle directly
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    rng = np.random.default_rng(11)
    S = []
    while len(S) < 64:
        b = int(rng.integers(0, w.B))
        if w.chunk_len[b]:
            S.append((b, int(rng.integers(0, w.Hq)), int(rng.integers(0, w.chunk_len[b]))))
    S = np.array(S, dtype=np.int64)
    Os, Ls = oracle.attention_rows(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q, w.prefix_len, w.Hkv, S)
    rows = torch.from_numpy(w.cu_q[S[:, 0]] + S[:, 2]).cuda()
    heads = torch.from_numpy(S[:, 1]).cuda()
    og = o[rows, heads].float().cpu().numpy()
    compare(w, og, Os, f"{name} fused")
    assert np.max(np.abs(lse[rows, heads].cpu().numpy() - Ls)) < 2e-2
    report(f"{name} fused {layout} (64 random rows)", error_stats(og, Os))
