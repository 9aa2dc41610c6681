"""The C-ABI library loads, exports every symbol include/cpa.h declares, and rejects invalid
arguments on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import sparse_attention_long_reduce_amd as cpa
from sparse_attention_long_reduce_amd import _lib

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "cpa.h")
DIAG_HEADER = os.path.join(INCLUDE, "cpa_diag.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cpa_[a-z0-9_]+)\s*\(", text)))


def test_every_header_is_covered():
    # each header under include/ is checked against a library below
    assert sorted(f for f in os.listdir(INCLUDE) if f.endswith(".h")) == ["cpa.h", "cpa_diag.h"]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libcpa.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"cpa_append_kv", "cpa_build_block_plans", "cpa_build_block_tables",
                          "cpa_build_block_tables_bits", "cpa_chunked_prefill", "cpa_chunked_prefill_direct",
                          "cpa_chunked_prefill_fp8kv", "cpa_chunked_prefill_fused", "cpa_chunked_prefill_fused_bits",
                          "cpa_chunked_prefill_split",
                          "cpa_chunked_prefill_split_static",
                          "cpa_chunked_prefill_vt", "cpa_split_workspace_bytes", "cpa_status_string", "cpa_version"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(_lib.EXPORTS) == set(names)


@pytest.fixture(scope="module")
def diag():
    if not os.path.exists(_lib.DIAG_LIB_PATH):
        pytest.fail("libcpa_diag.so is not built (run __graft_entry__.build())")
    return _lib.load_diag()


def test_diag_exports_every_declared_symbol(diag):
    names = declared_functions(DIAG_HEADER)
    assert set(names) == {"cpa_diag_mfma_loop", "cpa_diag_clock_rates"}
    for n in names:
        assert hasattr(diag, n), n
    assert set(_lib.DIAG_EXPORTS) == set(names)


def test_diag_validation(diag):
    import ctypes
    ml = diag.cpa_diag_mfma_loop
    assert ml(0, 512, 10, FAKE, FAKE, None) == 2
    assert ml(1, 32, 10, FAKE, FAKE, None) == 2
    assert ml(1, 576, 10, FAKE, FAKE, None) == 2
    assert ml(1, 100, 10, FAKE, FAKE, None) == 2
    assert ml(1, 512, 0, FAKE, FAKE, None) == 2
    assert ml(1, 512, 10 ** 7 + 1, FAKE, FAKE, None) == 2
    assert ml(1, 512, 10, None, FAKE, None) == 1
    assert ml(1, 512, 10, FAKE, None, None) == 1
    assert ml(1, 512, 10, FAKE, FAKE + 4, None) == 3
    x = ctypes.c_int(0)
    assert diag.cpa_diag_clock_rates(0, None, ctypes.byref(x)) == 1
    assert diag.cpa_diag_clock_rates(0, ctypes.byref(x), None) == 1


def test_status_strings(lib):
    for code in range(7):
        s = lib.cpa_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.cpa_status_string(99).decode() == "unknown status"
    assert lib.cpa_version() == 10000


NULL = None
FAKE = 0x1000  # never dereferenced: every call below fails validation before touching memory


def bt(lib, masks=FAKE, B=1, Hq=8, Hkv=2, nqb=4, nkvb=16, pb=FAKE, cb=FAKE, tab=FAKE, cap=16, cnt=FAKE):
    return lib.cpa_build_block_tables(masks, B, Hq, Hkv, nqb, nkvb, pb, cb, tab, cap, cnt, None)


def test_build_tables_validation(lib):
    assert bt(lib, Hkv=0) == 2
    assert bt(lib, Hq=6, Hkv=4) == 2
    assert bt(lib, B=-1) == 2
    assert bt(lib, nkvb=65537, cap=70000) == 2
    assert bt(lib, cap=15) == 5
    assert bt(lib, pb=NULL) == 1
    assert bt(lib, cnt=NULL) == 1
    assert bt(lib, masks=NULL) == 1
    assert bt(lib, tab=NULL) == 1
    assert bt(lib, B=0, masks=NULL, pb=NULL, cb=NULL, tab=NULL, cnt=NULL) == 0


def btb(lib, bits=FAKE, B=1, Hq=8, Hkv=2, nqb=4, nkvb=130, words=3, pb=FAKE, cb=FAKE, tab=FAKE, cap=130, cnt=FAKE):
    return lib.cpa_build_block_tables_bits(bits, B, Hq, Hkv, nqb, nkvb, words, pb, cb, tab, cap, cnt, None)


def test_build_tables_bits_validation(lib):
    assert btb(lib, words=2) == 2          # 130 blocks need 3 words per row
    assert btb(lib, words=-1) == 2
    assert btb(lib, Hq=6, Hkv=4) == 2
    assert btb(lib, nkvb=65537, cap=70000, words=1025) == 2
    assert btb(lib, cap=129) == 5
    assert btb(lib, bits=NULL) == 1
    assert btb(lib, cnt=NULL) == 1
    assert btb(lib, bits=FAKE + 4) == 3
    assert btb(lib, B=0, bits=NULL, pb=NULL, cb=NULL, tab=NULL, cnt=NULL) == 0


def pf(lib, q=FAKE, dtype=1, k=FAKE, v=FAKE, ps=8 * 64 * 128, hs=64 * 128, ts=128, npages=10, pm=FAKE,
       pms=16, tab=FAKE, cap=16, cnt=FAKE, cu=FAKE, pl=FAKE, B=1, Hq=32, Hkv=8, d=128, mcl=256,
       scale=0.0, o=FAKE, lse=NULL):
    return lib.cpa_chunked_prefill(q, dtype, k, v, ps, hs, ts, npages, pm, pms, tab, cap, cnt, cu, pl,
                                   B, Hq, Hkv, d, mcl, scale, o, lse, None)


def test_prefill_validation(lib):
    assert pf(lib, d=96) == 4
    assert pf(lib, d=256) == 4
    assert pf(lib, dtype=7) == 4
    assert pf(lib, Hq=30, Hkv=8) == 2  # Hq % Hkv != 0
    assert pf(lib, scale=-1.0) == 2
    assert pf(lib, scale=float("nan")) == 2
    assert pf(lib, scale=float("inf")) == 2
    assert pf(lib, ts=64) == 2
    assert pf(lib, hs=63 * 128) == 2
    assert pf(lib, ps=7 * 64 * 128) == 2
    assert pf(lib, pms=0) == 2
    assert pf(lib, q=NULL) == 1
    assert pf(lib, o=NULL) == 1
    assert pf(lib, pm=NULL) == 1
    assert pf(lib, tab=NULL) == 1
    assert pf(lib, q=FAKE + 8) == 3
    assert pf(lib, k=FAKE + 2) == 3
    assert pf(lib, ts=132, hs=64 * 132, ps=8 * 64 * 132) == 3    # bf16 row of 264 B
    assert pf(lib, B=0, q=NULL, k=NULL, v=NULL, pm=NULL, tab=NULL, cnt=NULL, cu=NULL, pl=NULL, o=NULL) == 0
    assert pf(lib, mcl=0, q=NULL) == 0
    # an empty pool with work to do: idle copy slots stage page 0, so it is refused
    assert pf(lib, npages=0) == 2
    assert pf(lib, npages=-1) == 2
    assert pf(lib, npages=0, B=0) == 0
    assert pfv(lib, npages=0) == 2
    assert pfs(lib, npages=0) == 2


def pfs(lib, dtype=1, total_q=256, split=4, ws=FAKE, ws_bytes=1 << 30, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ps=8 * 64 * 128, hs=64 * 128, ts=128, npages=10, pm=FAKE, pms=16,
             tab=FAKE, cap=16, cnt=FAKE, cu=FAKE, pl=FAKE, B=1, Hq=32, Hkv=8, d=128, mcl=256, scale=0.0,
             o=FAKE, lse=NULL)
    a.update(kw)
    return lib.cpa_chunked_prefill_split(a["q"], dtype, a["k"], a["v"], a["ps"], a["hs"], a["ts"], a["npages"],
                                         a["pm"], a["pms"], a["tab"], a["cap"], a["cnt"], a["cu"], a["pl"],
                                         a["B"], a["Hq"], a["Hkv"], a["d"], a["mcl"], a["scale"], a["o"],
                                         a["lse"], total_q, split, ws, ws_bytes, None)


def test_split_validation(lib):
    assert pfs(lib, split=0) == 2
    assert pfs(lib, total_q=-1) == 2
    assert pfs(lib, d=96) == 4                 # the checks of cpa_chunked_prefill come first
    assert pfs(lib, q=NULL) == 1
    assert pfs(lib, dtype=0) == 4              # fp32 has no split path (4 ranges of 4 pages)
    assert pfs(lib, ts=1 << 25, hs=64 << 25, ps=8 * (64 << 25)) == 4   # too wide for the split path
    assert pfs(lib, ws=NULL) == 1
    assert pfs(lib, ws=FAKE + 4) == 3
    need = lib.cpa_split_workspace_bytes(256, 32, 128, 16, 4)
    assert need == 4 * 256 * 32 * 129 * 4
    assert pfs(lib, ws_bytes=need - 1) == 5
    assert pfs(lib, B=0, q=NULL) == 0
    assert lib.cpa_split_workspace_bytes(256, 32, 128, 16, 16) == 0   # one range: no workspace
    assert lib.cpa_split_workspace_bytes(0, 32, 128, 16, 4) == 0


def pss(lib, dtype=1, total_q=256, split=4, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ps=8 * 64 * 128, hs=64 * 128, ts=128, npages=10, pm=FAKE, pms=16,
             tab=FAKE, cap=16, cnt=FAKE, cu=FAKE, pl=FAKE, B=1, Hq=32, Hkv=8, d=128, mcl=256, scale=0.0,
             o=FAKE, lse=NULL)
    a.update(kw)
    return lib.cpa_chunked_prefill_split_static(a["q"], dtype, a["k"], a["v"], a["ps"], a["hs"], a["ts"],
                                                a["npages"], a["pm"], a["pms"], a["tab"], a["cap"], a["cnt"], a["cu"],
                                                a["pl"], a["B"], a["Hq"], a["Hkv"], a["d"], a["mcl"], a["scale"],
                                                a["o"], a["lse"], total_q, split, None)


def test_split_static_validation(lib):
    # every refusal below happens on the host before the scratch array is looked up
    limit = 64 * 1024 * 1024
    assert pss(lib, split=0) == 2
    assert pss(lib, total_q=-1) == 2
    # 4 ranges x total_q x 32 heads x 129 floats: 1016 rows fit in 64 MiB, 1017 do not
    assert lib.cpa_split_workspace_bytes(1016, 32, 128, 16, 4) <= limit
    assert lib.cpa_split_workspace_bytes(1017, 32, 128, 16, 4) > limit
    assert pss(lib, total_q=1017) == 5
    assert pss(lib, total_q=1 << 20, split=1) == 5
    assert pss(lib, d=96) == 4
    assert pss(lib, q=NULL) == 1
    assert pss(lib, npages=0) == 2
    assert pss(lib, B=0, q=NULL) == 0


def pfv(lib, dtype=1, total_q=256, split=0, ws=NULL, ws_bytes=0, vps=8 * 128 * 64, vhs=128 * 64, vds=64, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ps=8 * 64 * 128, hs=64 * 128, ts=128, npages=10, pm=FAKE, pms=16,
             tab=FAKE, cap=16, cnt=FAKE, cu=FAKE, pl=FAKE, B=1, Hq=32, Hkv=8, d=128, mcl=256, scale=0.0,
             o=FAKE, lse=NULL)
    a.update(kw)
    return lib.cpa_chunked_prefill_vt(a["q"], dtype, a["k"], a["ps"], a["hs"], a["ts"], a["v"], vps, vhs, vds,
                                      a["npages"], a["pm"], a["pms"], a["tab"], a["cap"], a["cnt"], a["cu"],
                                      a["pl"], a["B"], a["Hq"], a["Hkv"], a["d"], a["mcl"], a["scale"], a["o"],
                                      a["lse"], total_q, split, ws, ws_bytes, None)


def pfu(lib, dtype=1, vdm=1, vps=8 * 128 * 64, vhs=128 * 64, vrs=64, masks=FAKE, nqb=4, nkvb=16, total_q=256,
        split=0, ws=NULL, ws_bytes=0, kvd=1, ks=1.0, vs=1.0, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ps=8 * 64 * 128, hs=64 * 128, ts=128, npages=10, pm=FAKE, pms=16,
             cu=FAKE, pl=FAKE, B=1, Hq=32, Hkv=8, d=128, mcl=256, scale=0.0, o=FAKE, lse=NULL)
    a.update(kw)
    return lib.cpa_chunked_prefill_fused(a["q"], dtype, a["k"], a["ps"], a["hs"], a["ts"], a["v"], vdm, vps, vhs,
                                         vrs, kvd, ks, vs, a["npages"], a["pm"], a["pms"], masks, nqb,
                                         nkvb, a["cu"], a["pl"], a["B"], a["Hq"], a["Hkv"], a["d"], a["mcl"],
                                         a["scale"], a["o"], a["lse"], total_q, split, ws, ws_bytes, None)


def test_fused_validation(lib):
    assert pfu(lib, vdm=2) == 2                       # V layout flag
    assert pfu(lib, nqb=-1) == 2
    assert pfu(lib, nkvb=-1) == 2
    assert pfu(lib, nkvb=65537) == 2                  # beyond CPA_MAX_KV_BLOCKS
    assert pfu(lib, masks=NULL) == 1
    assert pfu(lib, masks=NULL, nkvb=0, dtype=0) == 4   # no mask byte to read: NULL passes that check
    assert pfu(lib, dtype=0) == 4                     # bf16 only
    assert pfu(lib, d=96) == 4
    assert pfu(lib, vrs=1 << 25, vhs=128 << 25, vps=8 * (128 << 25)) == 4   # 32-bit offsets within a page
    assert pfu(lib, vrs=63) == 2                      # a dim row must hold the page's 64 tokens
    assert pfu(lib, vdm=0, vps=8 * 64 * 128, vhs=64 * 128, vrs=120) == 2    # a token row must hold d
    assert pfu(lib, vdm=0, vps=8 * 64 * 132, vhs=64 * 132, vrs=132) == 3    # 264-byte bf16 rows
    assert pfu(lib, q=NULL) == 1
    assert pfu(lib, cu=NULL) == 1
    assert pfu(lib, o=FAKE + 2) == 3
    assert pfu(lib, Hq=30) == 2                       # Hq % Hkv
    assert pfu(lib, npages=0) == 2
    assert pfu(lib, B=0, q=NULL, masks=NULL) == 0     # nothing to do
    assert pfu(lib, mcl=0) == 0
    # split-KV: ranges of nkvb_max ids, the checks of cpa_chunked_prefill_split
    assert pfu(lib, split=4) == 1                     # 4 ranges and no workspace
    assert pfu(lib, split=4, total_q=-1) == 2
    assert pfu(lib, split=4, ws=FAKE + 8, ws_bytes=1 << 30) == 3
    assert pfu(lib, split=4, ws=FAKE, ws_bytes=16) == 5
    assert lib.cpa_split_workspace_bytes(256, 32, 128, 16, 4) == 4 * 256 * 32 * 129 * 4
    assert pfu(lib, split=16, ws=NULL, masks=NULL, nkvb=0, dtype=0) == 4   # no mask columns: NULL masks pass, dtype still checked
    # the pools' element type: bf16, or fp8 with finite positive scales and 16-byte byte strides
    assert pfu(lib, kvd=0) == 4                       # fp32 pools
    assert pfu(lib, kvd=7) == 4
    assert pfu(lib, kvd=2, ks=0.0) == 2
    assert pfu(lib, kvd=2, vs=float("inf")) == 2
    assert pfu(lib, kvd=2, vs=float("nan")) == 2
    assert pfu(lib, kvd=2, ts=136, hs=64 * 136, ps=8 * 64 * 136) == 3   # fp8 strides are bytes
    assert pfu(lib, kvd=2, vrs=72, vhs=128 * 72, vps=8 * 128 * 72) == 3
    assert pfu(lib, kvd=2, split=4) == 1              # fp8 split: 4 ranges and no workspace
    assert pfu(lib, kvd=2, split=4, ws=FAKE, ws_bytes=16) == 5


def pfb(lib, masks=FAKE, nqb=4, nkvb=100, words=2, dtype=1, kvd=1, ks=1.0, vs=1.0, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ps=8 * 64 * 128, hs=64 * 128, ts=128, npages=10, pm=FAKE, pms=16,
             cu=FAKE, pl=FAKE, B=1, Hq=32, Hkv=8, d=128, mcl=256, scale=0.0, o=FAKE, lse=NULL)
    a.update(kw)
    return lib.cpa_chunked_prefill_fused_bits(a["q"], dtype, a["k"], a["ps"], a["hs"], a["ts"], a["v"], 1,
                                              8 * 128 * 64, 128 * 64, 64, kvd, ks, vs, a["npages"], a["pm"], a["pms"],
                                              masks, nqb,
                                              nkvb, words, a["cu"], a["pl"], a["B"], a["Hq"], a["Hkv"], a["d"],
                                              a["mcl"], a["scale"], a["o"], a["lse"], 256, 0, NULL, 0, None)


def test_fused_bits_validation(lib):
    assert pfb(lib, words=1) == 2                     # 100 blocks need two 64-bit words per row
    assert pfb(lib, nkvb=65537, words=1025) == 2
    assert pfb(lib, masks=NULL) == 1
    assert pfb(lib, masks=FAKE + 4) == 3              # 8-byte alignment
    assert pfb(lib, dtype=0) == 4
    assert pfb(lib, masks=NULL, nkvb=0, words=0, dtype=0) == 4   # nothing to read: NULL passes
    assert pfb(lib, q=NULL) == 1
    assert pfb(lib, B=0, q=NULL, masks=NULL) == 0
    assert pfb(lib, kvd=2, ks=-1.0) == 2
    assert pfb(lib, kvd=3) == 4


def test_vt_validation(lib):
    assert pfv(lib, vds=63) == 2                      # a dim row must hold the page's 64 tokens
    assert pfv(lib, vhs=127 * 64) == 2                # d dim rows per head
    assert pfv(lib, vps=7 * 128 * 64) == 2            # Hkv heads per page
    assert pfv(lib, vds=68, vhs=128 * 68, vps=8 * 128 * 68) == 3   # bf16 row of 136 B
    assert pfv(lib, ts=64) == 2                       # K is still checked
    assert pfv(lib, d=96) == 4
    assert pfv(lib, v=NULL) == 1
    assert pfv(lib, v=FAKE + 2) == 3
    # d = 64: rows of 64 tokens, 64 of them per head
    assert pfv(lib, d=64, ps=8 * 64 * 64, hs=64 * 64, ts=64, vps=8 * 64 * 64, vhs=64 * 64, vds=63) == 2
    # the split form: the split checks apply
    assert pfv(lib, split=4) == 1                     # no workspace
    assert pfv(lib, split=4, ws=FAKE, ws_bytes=1 << 30, dtype=0) == 4
    assert pfv(lib, split=4, ws=FAKE, ws_bytes=1 << 30, vds=1 << 25, vhs=128 << 25, vps=8 * (128 << 25)) == 4
    assert pfv(lib, split=4, ws=FAKE, ws_bytes=16, total_q=256) == 5
    assert pfv(lib, split=4, total_q=-1) == 2
    assert pfv(lib, B=0, q=NULL, k=NULL, v=NULL, pm=NULL, tab=NULL, cnt=NULL, cu=NULL, pl=NULL, o=NULL) == 0


def ap(lib, kn=FAKE, vn=FAKE, dtype=1, k=FAKE, ps=8 * 64 * 128, hs=64 * 128, ts=128, v=FAKE, vdm=0,
       vps=8 * 64 * 128, vhs=64 * 128, vrs=128, npages=10, pm=FAKE, pms=16, cu=FAKE, pl=FAKE, B=1, Hkv=8, d=128,
       mcl=256):
    return lib.cpa_append_kv(kn, vn, dtype, k, ps, hs, ts, v, vdm, vps, vhs, vrs, npages, pm, pms, cu, pl, B, Hkv,
                             d, mcl, None)


def test_append_validation(lib):
    assert ap(lib, d=96) == 4
    assert ap(lib, dtype=5) == 4
    assert ap(lib, dtype=2, ts=8, hs=64 * 8, ps=8 * 64 * 8) == 2   # fp8 rows still hold d values
    assert ap(lib, Hkv=0) == 2
    assert ap(lib, B=-1) == 2
    assert ap(lib, vdm=2) == 2
    assert ap(lib, ts=64) == 2
    assert ap(lib, vrs=64) == 2                       # token-major V rows hold d = 128 values
    assert ap(lib, vdm=1, vrs=63, vhs=128 * 64, vps=8 * 128 * 64) == 2
    assert ap(lib, vdm=1, vrs=64, vhs=127 * 64, vps=8 * 128 * 64) == 2
    assert ap(lib, pms=0) == 2
    assert ap(lib, kn=NULL) == 1
    assert ap(lib, v=NULL) == 1
    assert ap(lib, pm=NULL) == 1
    assert ap(lib, kn=FAKE + 4) == 3
    assert ap(lib, ts=132, hs=64 * 132, ps=8 * 64 * 132) == 3
    assert ap(lib, vdm=1, vrs=68, vhs=128 * 68, vps=8 * 128 * 68) == 3
    assert ap(lib, B=0, kn=NULL, vn=NULL, k=NULL, v=NULL, pm=NULL, cu=NULL, pl=NULL) == 0
    assert ap(lib, mcl=0, kn=NULL) == 0


def bp(lib, masks=FAKE, B=1, Hq=8, nqb=4, nkvb=16, pb=FAKE, cb=FAKE, plans=FAKE, cap=16, cnt=FAKE):
    return lib.cpa_build_block_plans(masks, B, Hq, nqb, nkvb, pb, cb, plans, cap, cnt, None)


def test_build_plans_validation(lib):
    assert bp(lib, B=-1) == 2
    assert bp(lib, nkvb=65537, cap=70000) == 2
    assert bp(lib, cap=15) == 5
    assert bp(lib, masks=NULL) == 1
    assert bp(lib, plans=NULL) == 1
    assert bp(lib, cnt=NULL) == 1
    assert bp(lib, B=0, masks=NULL, pb=NULL, cb=NULL, plans=NULL, cnt=NULL) == 0


def pd(lib, q=FAKE, dtype=1, k=FAKE, ps=8 * 64 * 128, hs=64 * 128, ts=128, v=FAKE, vps=8 * 128 * 64, vhs=128 * 64,
       vds=64, npages=10, pm=FAKE, pms=16, plans=FAKE, cap=16, cnt=FAKE, nqb=4, cu=FAKE, pl=FAKE, B=1, Hq=32, Hkv=8,
       d=128, mcl=256, scale=0.0, o=FAKE, lse=NULL):
    return lib.cpa_chunked_prefill_direct(q, dtype, k, ps, hs, ts, v, vps, vhs, vds, npages, pm, pms, plans, cap,
                                          cnt, nqb, cu, pl, B, Hq, Hkv, d, mcl, scale, o, lse, None)


def test_direct_validation(lib):
    assert pd(lib, dtype=0) == 4               # bf16 only
    assert pd(lib, d=96) == 4
    assert pd(lib, Hq=30) == 2
    assert pd(lib, nqb=3) == 2                 # plans must cover ceil(256 / 64) query blocks
    assert pd(lib, vds=63) == 2
    assert pd(lib, vhs=127 * 64) == 2
    assert pd(lib, ts=64) == 2
    assert pd(lib, scale=-1.0) == 2
    assert pd(lib, q=NULL) == 1
    assert pd(lib, plans=NULL) == 1
    assert pd(lib, cnt=NULL) == 1
    assert pd(lib, v=FAKE + 2) == 3
    assert pd(lib, vds=68, vhs=128 * 68, vps=8 * 128 * 68) == 3
    assert pd(lib, B=0, q=NULL, k=NULL, v=NULL, pm=NULL, plans=NULL, cnt=NULL, cu=NULL, pl=NULL, o=NULL) == 0


def pf8(lib, q=FAKE, k=FAKE, v=FAKE, ps=8 * 64 * 128, hs=64 * 128, ts=128, vdm=0, vps=8 * 64 * 128, vhs=64 * 128,
        vrs=128, ks=1.0, vs=1.0, npages=10, pm=FAKE, pms=16, tab=FAKE, cap=16, cnt=FAKE, cu=FAKE, pl=FAKE, B=1, Hq=32,
        Hkv=8, d=128, mcl=256, scale=0.0, o=FAKE, lse=NULL, tq=256, sp=0, ws=NULL, wsb=0):
    return lib.cpa_chunked_prefill_fp8kv(q, k, v, ps, hs, ts, vdm, vps, vhs, vrs, ks, vs, npages, pm, pms, tab, cap,
                                         cnt, cu, pl, B, Hq, Hkv, d, mcl, scale, o, lse, tq, sp, ws, wsb, None)


def test_fp8kv_validation(lib):
    assert pf8(lib, ks=0.0) == 2
    assert pf8(lib, vs=-1.0) == 2
    assert pf8(lib, ks=float("inf")) == 2
    assert pf8(lib, vs=float("nan")) == 2
    assert pf8(lib, vdm=3) == 2
    assert pf8(lib, d=96) == 4
    assert pf8(lib, ts=64) == 2
    assert pf8(lib, q=NULL) == 1
    assert pf8(lib, k=FAKE + 8) == 3
    assert pf8(lib, vdm=1, vrs=63, vhs=128 * 64, vps=8 * 128 * 64) == 2
    # fp8 strides are bytes: rows, heads and pages must start on 16-byte boundaries
    assert pf8(lib, ts=136, hs=64 * 136, ps=8 * 64 * 136) == 3
    assert pf8(lib, vdm=1, vrs=72, vhs=128 * 72, vps=8 * 128 * 72) == 3
    assert pf8(lib, vrs=136, vhs=64 * 136, vps=8 * 64 * 136) == 3
    assert pf8(lib, npages=0) == 2               # a call with work needs a non-empty pool
    # split-KV: the checks of cpa_chunked_prefill_split (ranges of 4 pages over a 16-entry table)
    assert pf8(lib, sp=4, tq=-1) == 2
    assert pf8(lib, sp=4) == 1                   # no workspace
    assert pf8(lib, sp=4, ws=FAKE + 8, wsb=1 << 30) == 3
    assert pf8(lib, sp=4, ws=FAKE, wsb=16) == 5  # workspace too small
    need = lib.cpa_split_workspace_bytes(256, 32, 128, 16, 4)
    assert need == 4 * 256 * 32 * 129 * 4
    assert pf8(lib, sp=4, ws=FAKE, wsb=need - 1) == 5
    big = 1 << 25                                # rows past the split kernel's 32-bit offsets
    assert pf8(lib, sp=4, ws=FAKE, wsb=need, ts=big, hs=64 * big, ps=8 * 64 * big) == 4
    assert pf8(lib, B=0, q=NULL, k=NULL, v=NULL, pm=NULL, tab=NULL, cnt=NULL, cu=NULL, pl=NULL, o=NULL) == 0


def test_split_planner():
    # one KV group of a 128K context (4 query heads, 2048-row chunk): 32 tiles on 256 CUs
    assert cpa.prefill_tiles(1, 4, 1, 2048) == 32
    assert cpa.plan_split_pages(1, 4, 1, 2048, 2048, 256) == 256
    # the whole layer (32 heads, 8 groups) already has a tile per CU
    assert cpa.prefill_tiles(1, 32, 8, 2048) == 256
    assert cpa.plan_split_pages(1, 32, 8, 2048, 2048, 256) == 0
    # G = 1 packs 4 query blocks, G = 8 splits the heads in two, G = 3 / 7 tiles span query blocks
    assert cpa.prefill_tiles(2, 8, 8, 300) == 2 * 8 * 2 * 1
    assert cpa.prefill_tiles(1, 16, 2, 128) == 1 * 2 * 2 * 2
    assert cpa.prefill_tiles(1, 24, 8, 2048) == 8 * 24          # 32 query blocks x 3 heads / 4
    assert cpa.prefill_tiles(1, 28, 4, 2048) == 4 * 56          # 32 x 7 / 4
    assert cpa.prefill_tiles(1, 5, 1, 100) == 3                 # 2 query blocks x 5 heads -> 10 pairs
    assert cpa.plan_split_pages(1, 4, 1, 64, 1, 256) == 0


def test_python_layer_rejects_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        cpa.build_block_tables(torch.zeros((1, 8, 4, 16), dtype=torch.uint8),
                               torch.zeros(1, dtype=torch.int32), torch.zeros(1, dtype=torch.int32), 2)


def test_attention_flops_matches_oracle_visible_counts():
    import numpy as np
    import oracle
    from workloads import make_workload
    from workloads.configs import mask_bernoulli
    w = make_workload("f", [128, 320, 0], [128, 100, 64], 8, 2, 8, "f32",
                      lambda rng, *a: mask_bernoulli(rng, *a, p=0.2, local=1), 3)
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    _, _, NV = oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q,
                                      w.prefix_len, w.Hkv, return_nvis=True)
    assert cpa.attention_flops(T, C, w.prefix_len, w.chunk_len, w.Hq, w.Hkv, w.d) == 4 * w.d * int(NV.sum())


def test_plan_flops_matches_oracle_visible_counts():
    import numpy as np
    import oracle
    from workloads import make_workload
    from workloads.configs import mask_bernoulli
    w = make_workload("pf", [128, 320, 0], [128, 100, 64], 8, 2, 8, "f32",
                      lambda rng, *a: mask_bernoulli(rng, *a, p=0.3, local=1), 4)
    P, C = oracle.block_plans(w.masks, w.prefix_blocks, w.chunk_blocks, w.nkvb_max)
    pairs = 0
    for b in range(w.B):
        for h in range(w.Hq):
            for r in range(int(w.chunk_len[b])):
                qi = r // 64
                for kb in P[b, h, qi, :C[b, h, qi]].tolist():
                    pairs += sum(1 for t in range(64 * kb, 64 * kb + 64) if t <= int(w.prefix_len[b]) + r)
    assert cpa.plan_flops(P, C, w.prefix_len, w.chunk_len, w.d) == 4 * w.d * pairs


def test_size_caps(lib):
    # strides past 2^40 elements, more than 65536 heads, or a grid past INT_MAX workgroups are
    # refused on the host: no size product the checks or the kernels form can overflow
    big = (1 << 40) + 64
    assert pf(lib, ts=big, hs=64 * big, ps=8 * 64 * big) == 2
    assert pf(lib, Hq=4 * 32768, Hkv=32768) == 2
    assert pf(lib, B=1 << 29) == 2                      # B * Hkv = 2^32 KV groups
    assert pf(lib, B=1 << 26, mcl=1 << 20) == 2         # 2^29 groups x 4096 query tiles
    assert pfs(lib, B=1 << 20, mcl=1 << 12) == 2        # 2^23 groups x 64 tiles fit; x 4 ranges do not
    assert ap(lib, ts=big, hs=64 * big, ps=8 * 64 * big) == 2
    assert ap(lib, Hkv=65537) == 2
    assert ap(lib, B=1 << 20, mcl=1 << 20) == 2         # 2^20 sequences x 2^14 chunk pages x 8 groups
