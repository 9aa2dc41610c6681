"""Pins for the CPU oracle: each test checks it against something other than itself.

Source of the properties: "CompactAttention: Accelerating Chunked Prefill with
Block-Union KV Selection", abstract (Q-block union, intra-group union, minimal tables that keep
every selected KV block, attention over the selected blocks read in place), plus textbook
attention (torch SDPA, closed forms, the log-sum-exp merge identity) and brute-force loops.
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from workloads import BLOCK, make_workload, make_config
from workloads.configs import mask_all, mask_bernoulli, mask_stripes, mask_structured

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def tables_of(w, cap=None):
    cap = w.nkvb_max if cap is None else cap
    return oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, cap)


def run_oracle(w, T=None, C=None, **kw):
    if T is None:
        T, C = tables_of(w)
    return oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q,
                                  w.prefix_len, w.Hkv, **kw)


def small(seed, G=2, Hkv=2, d=16, prefix=(128, 320), chunk=(128, 64), p=0.15, noise=0.0,
          values=False, fn=None, dtype="f32"):
    fn = fn or (lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=1))
    return make_workload("small", list(prefix), list(chunk), G * Hkv, Hkv, d, dtype, fn, seed,
                         noncausal_noise=noise, mask_values=values)


def contiguous_kv(w, b, g):
    """Logical K/V of sequence b, group g, in token order (test-side gather via the page map)."""
    L = int(w.prefix_len[b] + w.chunk_len[b])
    nb = (L + BLOCK - 1) // BLOCK
    phys = w.page_map[b, :nb]
    return (w.k_pages[phys, g].reshape(nb * BLOCK, w.d)[:L].astype(np.float64),
            w.v_pages[phys, g].reshape(nb * BLOCK, w.d)[:L].astype(np.float64))


# ------------------------------------------------------------------------------------------
# tables
# ------------------------------------------------------------------------------------------

def loop_tables(w):
    """Pure-Python loops straight from the definition: kb is in group g's table iff some head
    of g and some Q-block qi of the chunk select it and it is causally reachable from qi."""
    B, Hq, _, _ = w.masks.shape
    G = Hq // w.Hkv
    out = {}
    for b in range(B):
        qb0, nqb = int(w.prefix_blocks[b]), int(w.chunk_blocks[b])
        for g in range(w.Hkv):
            sel = []
            for kb in range(qb0 + nqb):
                hit = False
                for h in range(g * G, (g + 1) * G):
                    for qi in range(nqb):
                        if kb <= qb0 + qi and w.masks[b, h, qi, kb] != 0:
                            hit = True
                if hit:
                    sel.append(kb)
            out[(b, g)] = sel
    return out


@pytest.mark.parametrize("seed,G,noise,values", [(1, 1, 0.0, False), (2, 2, 0.3, False),
                                                 (3, 4, 0.5, True), (4, 4, 0.0, True)])
def test_tables_equal_loop_definition(seed, G, noise, values):
    w = small(seed, G=G, noise=noise, values=values)
    T, C = tables_of(w, cap=w.nkvb_max + 3)
    ref = loop_tables(w)
    for (b, g), sel in ref.items():
        assert C[b, g] == len(sel)
        assert list(T[b, g, :C[b, g]]) == sel
        assert np.all(T[b, g, C[b, g]:] == -1)


@st.composite
def raw_mask_inputs(draw):
    """Byte masks drawn directly, with nonzero entries anywhere: past the causal limit, in padding
    rows past a sequence's query blocks and in padding columns past its KV extent."""
    B = draw(st.integers(1, 3))
    G, Hkv = draw(st.sampled_from([1, 2, 3, 4])), draw(st.integers(1, 3))
    nqb_max = draw(st.integers(1, 5))
    cb = [draw(st.integers(0, nqb_max)) for _ in range(B)]
    pb = [draw(st.integers(0, 6)) for _ in range(B)]
    nkvb_max = max(1, max(p + c for p, c in zip(pb, cb)) + draw(st.integers(0, 3)))
    density = draw(st.floats(0.0, 1.0))
    rng = np.random.default_rng(draw(st.integers(0, 2 ** 31 - 1)))
    shape = (B, G * Hkv, nqb_max, nkvb_max)
    masks = np.where(rng.random(shape) < density, rng.integers(1, 256, size=shape), 0).astype(np.uint8)
    return SimpleNamespace(masks=masks, prefix_blocks=np.array(pb, np.int32), chunk_blocks=np.array(cb, np.int32),
                           Hkv=Hkv)


@settings(max_examples=200, deadline=None)
@given(raw_mask_inputs())
def test_tables_equal_loop_definition_on_drawn_masks(w):
    nkvb_max = w.masks.shape[3]
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, nkvb_max)
    for (b, g), sel in loop_tables(w).items():
        assert C[b, g] == len(sel)
        assert list(T[b, g, :C[b, g]]) == sel
        assert np.all(T[b, g, C[b, g]:] == -1)


def test_tables_superset_and_minimal():
    w = small(7, G=4, Hkv=2, prefix=(0, 640, 192), chunk=(192, 128, 448), p=0.05, noise=0.2)
    T, C = tables_of(w)
    G = w.G
    for b in range(w.B):
        qb0, nqb = int(w.prefix_blocks[b]), int(w.chunk_blocks[b])
        for g in range(w.Hkv):
            table = set(T[b, g, :C[b, g]].tolist())
            assert list(T[b, g, :C[b, g]]) == sorted(table)          # strictly ascending
            witnessed = set()
            for h in range(g * G, (g + 1) * G):
                for qi in range(nqb):
                    for kb in range(qb0 + qi + 1):
                        if w.masks[b, h, qi, kb]:
                            assert kb in table                        # superset: nothing dropped
                            witnessed.add(kb)
            assert table == witnessed                                 # minimal: every entry has a witness


def test_tables_special_cases():
    ones = small(5, G=4, fn=lambda rng, *a: mask_all(rng, *a, value=1), noise=0.4)
    T, C = tables_of(ones)
    for b in range(ones.B):
        n = int(ones.prefix_blocks[b] + ones.chunk_blocks[b])
        for g in range(ones.Hkv):
            assert C[b, g] == n and list(T[b, g, :n]) == list(range(n))
    zero = small(6, G=4, fn=lambda rng, *a: mask_all(rng, *a, value=0), noise=0.4)
    T, C = tables_of(zero)
    assert np.all(C == 0) and np.all(T == -1)
    # one head per group and a single Q-block: the table is that head's (clipped) mask row
    one = small(8, G=1, Hkv=3, prefix=(448,), chunk=(64,), p=0.4, noise=0.3)
    T, C = tables_of(one)
    for g in range(3):
        row = np.nonzero(one.masks[0, g, 0, :int(one.prefix_blocks[0]) + 1])[0]
        assert list(T[0, g, :C[0, g]]) == list(row)


def test_tables_partial_bitset_word():
    # 70 KV blocks: a length that is not a multiple of 64
    w = small(9, G=4, Hkv=2, prefix=(64 * 66,), chunk=(256,), p=0.05, noise=0.1)
    T, C = tables_of(w)
    ref = loop_tables(w)
    for (b, g), sel in ref.items():
        assert list(T[b, g, :C[b, g]]) == sel


def test_tables_capacity_checked():
    w = small(10, G=2)
    with pytest.raises(ValueError):
        tables_of(w, cap=3)


# ------------------------------------------------------------------------------------------
# attention
# ------------------------------------------------------------------------------------------

def sdpa_dense(w, token_mask=None):
    """torch SDPA in float64 on contiguous K/V with an explicit boolean mask; with
    token_mask=None the mask is plain bottom-right causal (key position <= query position)."""
    out = np.zeros(w.q.shape, dtype=np.float64)
    lse = np.zeros((w.Hq, w.q.shape[0]), dtype=np.float64)
    for b in range(w.B):
        P, Cn = int(w.prefix_len[b]), int(w.chunk_len[b])
        q0 = int(w.cu_q[b])
        for h in range(w.Hq):
            g = h // w.G
            K, V = contiguous_kv(w, b, g)
            Q = w.q[q0:q0 + Cn, h].astype(np.float64)
            allowed = np.arange(P + Cn)[None, :] <= (P + np.arange(Cn))[:, None]
            if token_mask is not None:
                allowed = allowed & token_mask(b, h)
            Qt, Kt, Vt = (torch.from_numpy(x)[None, None] for x in (Q, K, V))
            m = torch.from_numpy(allowed)[None, None]
            o = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=m,
                                                                 scale=1 / math.sqrt(w.d))
            out[q0:q0 + Cn, h] = o[0, 0].numpy()
            s = (torch.from_numpy(Q) @ torch.from_numpy(K).T) / math.sqrt(w.d)
            s = s.masked_fill(~torch.from_numpy(allowed), -math.inf)
            lse[h, q0:q0 + Cn] = torch.logsumexp(s, dim=1).numpy()
    return out, lse


@pytest.mark.parametrize("chunk", [(192, 64), (150, 37)])
def test_all_ones_is_dense_causal_attention(chunk):
    w = small(11, G=2, Hkv=2, d=32, prefix=(128, 320), chunk=chunk,
              fn=lambda rng, *a: mask_all(rng, *a, value=1))
    O, L = run_oracle(w)
    Od, Ld = sdpa_dense(w)
    assert np.max(np.abs(O - Od)) < 1e-12
    assert np.max(np.abs(L - Ld)) < 1e-12


def test_union_of_qblock_constant_group_shared_masks_is_block_sparse_attention():
    # masks shared by a group's heads and constant over Q-blocks: the union adds nothing, so the
    # result equals per-query block-sparse attention with each head's own mask
    def fn(rng, Hq, Hkv, qb0, nqb, nkvb):
        m = mask_stripes(rng, Hq, Hkv, qb0, nqb, nkvb, p=0.3, shared_per_group=True)
        s = rng.random((Hkv, nkvb)) < 0.3
        s[:, 0] = True
        return np.broadcast_to(np.repeat(s, Hq // Hkv, axis=0)[:, None, :], m.shape).copy()
    w = small(12, G=4, Hkv=2, d=16, prefix=(256, 512), chunk=(128, 192), fn=fn)
    T, C = tables_of(w)
    O, _ = run_oracle(w, T, C)

    def token_mask(b, h):
        P, Cn = int(w.prefix_len[b]), int(w.chunk_len[b])
        blk = np.zeros((Cn, P + Cn), dtype=bool)
        for r in range(Cn):
            qi = r // BLOCK
            sel = np.nonzero(w.masks[b, h, qi, :(P + Cn + BLOCK - 1) // BLOCK])[0]
            for kb in sel:
                blk[r, kb * BLOCK:(kb + 1) * BLOCK] = True
        return blk
    Os, _ = sdpa_dense(w, token_mask)
    assert np.max(np.abs(O - Os)) < 1e-12


def brute_force(w, T, C):
    """Per (query, key token) loops: key t is used by row (b, h, r) iff its block is in group
    h // G's table and t <= prefix + r; two-pass softmax with math.exp."""
    O = np.zeros(w.q.shape)
    scale = 1 / math.sqrt(w.d)
    for b in range(w.B):
        P, Cn, q0 = int(w.prefix_len[b]), int(w.chunk_len[b]), int(w.cu_q[b])
        for h in range(w.Hq):
            g = h // w.G
            table = set(T[b, g, :C[b, g]].tolist())
            for r in range(Cn):
                p = P + r
                q = [float(x) for x in w.q[q0 + r, h]]
                keys = []
                for t in range(P + Cn):
                    if t // BLOCK in table and t <= p:
                        page = int(w.page_map[b, t // BLOCK])
                        k = w.k_pages[page, g, t % BLOCK]
                        keys.append((scale * sum(qq * float(kk) for qq, kk in zip(q, k)), page, t % BLOCK))
                if not keys:
                    continue
                m = max(s for s, _, _ in keys)
                den = sum(math.exp(s - m) for s, _, _ in keys)
                for c in range(w.d):
                    O[q0 + r, h, c] = sum(math.exp(s - m) * float(w.v_pages[pg, g, tt, c])
                                          for s, pg, tt in keys) / den
    return O


@pytest.mark.parametrize("chunk", [(64, 128), (23, 100)])
def test_brute_force_tiny(chunk):
    w = small(13, G=2, Hkv=2, d=4, prefix=(128, 64), chunk=chunk, p=0.2)
    T, C = tables_of(w)
    O, _ = run_oracle(w, T, C)
    Ob = brute_force(w, T, C)
    assert np.max(np.abs(O - Ob)) < 1e-12


def test_brute_force_tables_with_holes():
    # sparse masks with one head per group so that tables keep holes
    w = small(14, G=1, Hkv=2, d=4, prefix=(256,), chunk=(64,), p=0.1)
    T, C = tables_of(w)
    assert np.all(C < w.prefix_blocks[0] + w.chunk_blocks[0])
    O, _ = run_oracle(w, T, C)
    assert np.max(np.abs(O - brute_force(w, T, C))) < 1e-12


def test_closed_forms():
    w = small(15, G=2, Hkv=2, d=8, prefix=(192,), chunk=(128,), p=0.3)
    T, C = tables_of(w)
    # V constant -> O equals that constant
    w.v_pages[:] = 0.375
    O, _ = run_oracle(w, T, C)
    assert np.max(np.abs(O - 0.375)) < 1e-14
    # q = 0 -> O is the plain mean of the visible V rows
    w2 = small(16, G=2, Hkv=2, d=8, prefix=(192,), chunk=(128,), p=0.3)
    T2, C2 = tables_of(w2)
    w2.q[:] = 0
    O2, L2 = run_oracle(w2, T2, C2)
    for h in range(w2.Hq):
        g = h // w2.G
        for r in range(int(w2.chunk_len[0])):
            p = int(w2.prefix_len[0]) + r
            rows = [w2.v_pages[w2.page_map[0, t // BLOCK], g, t % BLOCK].astype(np.float64)
                    for t in range(p + 1) if t // BLOCK in set(T2[0, g, :C2[0, g]].tolist())]
            assert np.max(np.abs(O2[r, h] - np.mean(rows, axis=0))) < 1e-13
            assert abs(L2[h, r] - math.log(len(rows))) < 1e-12
    # exactly one visible key: first row of a chunk with no prefix sees only token 0
    w3 = make_workload("one", [0], [64], 4, 2, 8, "f32",
                       lambda rng, *a: mask_all(rng, *a, value=1), 17)
    T3, C3 = tables_of(w3)
    O3, L3 = run_oracle(w3, T3, C3)
    for h in range(4):
        v0 = w3.v_pages[w3.page_map[0, 0], h // 2, 0]
        k0 = w3.k_pages[w3.page_map[0, 0], h // 2, 0].astype(np.float64)
        assert np.max(np.abs(O3[0, h] - v0)) == 0
        assert abs(L3[h, 0] - float(w3.q[0, h].astype(np.float64) @ k0) / math.sqrt(8)) < 1e-13


def test_lse_merge_identity():
    w = small(18, G=2, Hkv=2, d=16, prefix=(320, 128), chunk=(128, 192), p=0.3)
    T, C = tables_of(w)
    O, L = run_oracle(w, T, C)
    # split each table into its even- and odd-indexed entries
    parts = []
    for sl in (slice(0, None, 2), slice(1, None, 2)):
        Tp = np.full_like(T, -1)
        Cp = np.zeros_like(C)
        for b in range(w.B):
            for g in range(w.Hkv):
                ids = T[b, g, :C[b, g]][sl]
                Tp[b, g, :len(ids)] = ids
                Cp[b, g] = len(ids)
        parts.append(run_oracle(w, Tp, Cp))
    (O1, L1), (O2, L2) = parts
    Lm = np.logaddexp(L1, L2)
    w1 = np.exp(L1 - Lm).T[:, :, None]
    w2 = np.exp(L2 - Lm).T[:, :, None]
    assert np.max(np.abs(w1 * O1 + w2 * O2 - O)) < 1e-12
    assert np.max(np.abs(Lm - L)) < 1e-12


def test_page_permutation_invariance():
    w = small(19, G=2, Hkv=2, d=16, prefix=(256, 64), chunk=(128, 128), p=0.3)
    T, C = tables_of(w)
    O, L = run_oracle(w, T, C)
    rng = np.random.default_rng(0)
    perm = rng.permutation(w.n_pages)           # new physical slot of each old page
    k2 = np.empty_like(w.k_pages)
    v2 = np.empty_like(w.v_pages)
    k2[perm] = w.k_pages
    v2[perm] = w.v_pages
    pm2 = perm[w.page_map].astype(np.int32)
    O2, L2 = oracle.paged_attention(w.q, k2, v2, pm2, T, C, w.cu_q, w.prefix_len, w.Hkv)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_rows_entry_matches_full():
    w = small(20, G=4, Hkv=2, d=16, prefix=(384, 0), chunk=(128, 256), p=0.1)
    T, C = tables_of(w)
    O, L = run_oracle(w, T, C)
    rng = np.random.default_rng(1)
    samples = []
    for _ in range(60):
        b = int(rng.integers(0, w.B))
        samples.append((b, int(rng.integers(0, w.Hq)), int(rng.integers(0, w.chunk_len[b]))))
    Os, Ls = oracle.attention_rows(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q,
                                   w.prefix_len, w.Hkv, samples)
    for i, (b, h, r) in enumerate(samples):
        row = int(w.cu_q[b]) + r
        assert np.max(np.abs(Os[i] - O[row, h])) < 1e-13
        assert abs(Ls[i] - L[h, row]) < 1e-12


def test_block_attribution_oracle():
    # V one-hot by block: channel kb % d carries the softmax mass of block kb
    w = small(21, G=2, Hkv=2, d=16, prefix=(512,), chunk=(128,), p=0.2)
    for kb in range(w.page_map.shape[1]):
        page = w.page_map[0, kb]
        w.v_pages[page] = 0
        w.v_pages[page, :, :, kb % w.d] = 1
    T, C = tables_of(w)
    O, _ = run_oracle(w, T, C)
    assert np.max(np.abs(O.sum(axis=2) - 1)) < 1e-13
    for h in range(w.Hq):
        g = h // w.G
        for r in range(int(w.chunk_len[0])):
            qi_abs = int(w.prefix_blocks[0]) + r // BLOCK
            vis = {int(kb) % w.d for kb in T[0, g, :C[0, g]] if kb <= qi_abs}
            assert set(np.nonzero(O[r, h] > 0)[0].tolist()) == vis


def test_empty_table_row_is_zero():
    w = small(22, G=2, Hkv=2, d=8, fn=lambda rng, *a: mask_all(rng, *a, value=0))
    O, L = run_oracle(w)
    assert np.all(O == 0) and np.all(np.isneginf(L))


def test_nvis_counts():
    w = small(23, G=2, Hkv=2, d=8, prefix=(128,), chunk=(128,),
              fn=lambda rng, *a: mask_all(rng, *a, value=1))
    _, _, NV = run_oracle(w, return_nvis=True)
    assert np.array_equal(NV[:, 0], 128 + 1 + np.arange(128))


# ------------------------------------------------------------------------------------------
# generators
# ------------------------------------------------------------------------------------------

def test_generator_determinism_and_shapes():
    a = make_config("c1_tiny_f32")
    b = make_config("c1_tiny_f32")
    assert np.array_equal(a.masks, b.masks) and np.array_equal(a.q, b.q)
    assert np.array_equal(a.k_pages, b.k_pages) and np.array_equal(a.page_map, b.page_map)
    assert a.q.shape == (256, 8, 64) and a.k_pages.shape[1:] == (2, 64, 64)
    assert a.n_pages == 20 and len(set(a.page_map[0].tolist())) == 16
    assert a.poison_page not in set(a.page_map[0].tolist())
    c = make_config("c1_tiny_f32", seed=5)
    assert not np.array_equal(a.q, c.q)
    # masks: causal-only, sink and diagonal forced
    qb0 = 12
    for qi in range(4):
        assert np.all(a.masks[0, :, qi, qb0 + qi + 1:] == 0)
        assert np.all(a.masks[0, :, qi, 0] == 1) and np.all(a.masks[0, :, qi, qb0 + qi] == 1)


def test_bf16_rounding_is_exact_bf16():
    w = make_workload("t", [64], [64], 2, 1, 8, "bf16", lambda rng, *a: mask_all(rng, *a, value=1), 3)
    for x in (w.q, w.k_pages, w.v_pages):
        t = torch.from_numpy(x)
        assert torch.equal(t.to(torch.bfloat16).to(torch.float32), t)


def test_structured_mask_shape_and_density():
    # the 128K generator on a reduced width keeps its pattern rules
    import numpy.random as npr
    m = mask_structured(npr.default_rng(0), 4, 1, 100, 8, 108)
    assert m.shape == (4, 8, 108)
    assert np.all(m[:, :, 0])
    for qi in range(8):
        assert np.all(m[:, qi, 100 + qi - 3:100 + qi + 1])


# ---- KV append ---------------------------------------------------------------------------------

def test_append_kv_worked_example():
    # two sequences, one KV head, d = 2, four pages.  Sequence 0: prefix 64, chunk of 3 rows;
    # logical block 1 is page 0, so its rows land in page 0 slots 0..2.  Sequence 1: prefix 0,
    # chunk of 2 rows; block 0 is page 3.
    k_new = np.array([[[1, 2]], [[3, 4]], [[5, 6]], [[7, 8]], [[9, 10]]], dtype=np.float64)
    v_new = -k_new
    kp = np.zeros((4, 1, 64, 2))
    vp = np.zeros((4, 1, 64, 2))
    page_map = np.array([[2, 0], [3, 1]], dtype=np.int32)
    cu = np.array([0, 3, 5], dtype=np.int32)
    P = np.array([64, 0], dtype=np.int32)
    k2, v2 = oracle.append_kv(k_new, v_new, kp, vp, page_map, cu, P)
    expect = np.zeros((4, 1, 64, 2))
    expect[0, 0, 0] = [1, 2]
    expect[0, 0, 1] = [3, 4]
    expect[0, 0, 2] = [5, 6]
    expect[3, 0, 0] = [7, 8]
    expect[3, 0, 1] = [9, 10]
    assert np.array_equal(k2, expect) and np.array_equal(v2, -expect)
    assert not kp.any()   # inputs untouched


@pytest.mark.parametrize("seed", [0, 1])
def test_append_kv_reads_back_and_touches_nothing_else(seed):
    rng = np.random.default_rng(seed)
    w = make_workload("app", [0, 128, 640], [100, 64, 200], 8, 2, 16, "f32",
                      lambda r, *a: mask_all(r, *a, value=1), seed)
    k_new = rng.standard_normal((w.q.shape[0], w.Hkv, w.d)).astype(w.k_pages.dtype)
    v_new = rng.standard_normal((w.q.shape[0], w.Hkv, w.d)).astype(w.v_pages.dtype)
    pm = w.page_map.copy()
    pm[2, (640 + 150) // 64] = -1             # one unresolved page: its rows are dropped
    k2, v2 = oracle.append_kv(k_new, v_new, w.k_pages, w.v_pages, pm, w.cu_q, w.prefix_len)
    written = np.zeros(w.k_pages.shape[:1] + w.k_pages.shape[2:3], dtype=bool)   # [page][slot]
    for b in range(w.B):
        pos = w.prefix_len[b] + np.arange(w.chunk_len[b])
        pages = pm[b, pos // 64]
        ok = pages >= 0
        rows = w.cu_q[b] + np.arange(w.chunk_len[b])
        # read back through (page, slot) of each logical position, all heads at once
        assert np.array_equal(k2[pages[ok], :, pos[ok] % 64], k_new[rows[ok]])
        assert np.array_equal(v2[pages[ok], :, pos[ok] % 64], v_new[rows[ok]])
        written[pages[ok], pos[ok] % 64] = True
        assert (~ok).sum() == (64 if b == 2 else 0)
    keep = ~written
    assert np.array_equal(k2.transpose(0, 2, 1, 3)[keep], w.k_pages.transpose(0, 2, 1, 3)[keep])
    assert np.array_equal(v2.transpose(0, 2, 1, 3)[keep], w.v_pages.transpose(0, 2, 1, 3)[keep])


# ---- bit-packed masks ---------------------------------------------------------------------------

def test_unpack_mask_bits_worked_example():
    # two words: word 0 = bits 0, 1 and 63 set; word 1 = bit 5 set (block 69); 72 blocks
    w = np.zeros((1, 1, 1, 2), dtype=np.uint64)
    w[0, 0, 0, 0] = np.uint64((1 << 0) | (1 << 1) | (1 << 63))
    w[0, 0, 0, 1] = np.uint64(1 << 5) | np.uint64(1 << 20)   # bit 20 = block 84: past 72, dropped
    m = oracle.unpack_mask_bits(w, 72)
    assert m.shape == (1, 1, 1, 72)
    assert list(np.nonzero(m[0, 0, 0])[0]) == [0, 1, 63, 69]


def test_unpack_mask_bits_matches_per_bit_loop():
    from workloads.configs import pack_mask_bits
    rng = np.random.default_rng(3)
    masks = (rng.random((2, 3, 4, 150)) < 0.3).astype(np.uint8) * rng.integers(1, 256, (2, 3, 4, 150), dtype=np.uint8)
    bits = pack_mask_bits(masks)
    assert bits.shape == (2, 3, 4, 3) and bits.dtype == np.uint64
    for idx in np.ndindex(2, 3, 4):
        for kb in range(150):
            word = int(bits[idx][kb // 64])
            assert ((word >> (kb % 64)) & 1) == (masks[idx][kb] != 0)
    assert np.array_equal(oracle.unpack_mask_bits(bits, 150), masks != 0)
    T1, C1 = oracle.block_union_tables(masks, np.array([1, 0], np.int32), np.array([2, 4], np.int32), 3, 150)
    T2, C2 = oracle.block_union_tables_bits(bits, 150, np.array([1, 0], np.int32), np.array([2, 4], np.int32), 3)
    assert np.array_equal(T1, T2) and np.array_equal(C1, C2)


# ---- direct block-sparse baseline ----------------------------------------------------------------

@pytest.mark.parametrize("seed,noise", [(21, 0.0), (22, 0.4)])
def test_block_plans_equal_loop_definition(seed, noise):
    w = small(seed, G=2, Hkv=2, d=8, prefix=(128, 0, 640), chunk=(192, 37, 100), p=0.3, noise=noise, values=True)
    plans, counts = oracle.block_plans(w.masks, w.prefix_blocks, w.chunk_blocks, w.nkvb_max + 3)
    for b in range(w.B):
        for h in range(w.Hq):
            for qi in range(w.nqb_max):
                expect = []
                if qi < w.chunk_blocks[b]:
                    for kb in range(w.nkvb_max):
                        if w.masks[b, h, qi, kb] != 0 and kb <= w.prefix_blocks[b] + qi:
                            expect.append(kb)
                assert counts[b, h, qi] == len(expect)
                assert plans[b, h, qi].tolist() == expect + [-1] * (w.nkvb_max + 3 - len(expect))


@settings(max_examples=200, deadline=None)
@given(raw_mask_inputs())
def test_block_plans_equal_loop_definition_on_drawn_masks(w):
    B, Hq, nqb_max, nkvb_max = w.masks.shape
    plans, counts = oracle.block_plans(w.masks, w.prefix_blocks, w.chunk_blocks, nkvb_max)
    for b in range(B):
        for h in range(Hq):
            for qi in range(nqb_max):
                expect = [kb for kb in range(nkvb_max) if qi < w.chunk_blocks[b] and w.masks[b, h, qi, kb] != 0
                          and kb <= w.prefix_blocks[b] + qi]
                assert counts[b, h, qi] == len(expect)
                assert plans[b, h, qi].tolist() == expect + [-1] * (nkvb_max - len(expect))


def test_block_plans_one_head_one_block_is_the_union_table():
    # G = 1 and a one-block chunk: nothing to union, the plan is the group's table
    w = small(23, G=1, Hkv=3, d=8, prefix=(256, 64), chunk=(64, 50), p=0.3)
    plans, counts = oracle.block_plans(w.masks, w.prefix_blocks, w.chunk_blocks, w.nkvb_max)
    T, C = tables_of(w)
    assert np.array_equal(plans[:, :, 0], T) and np.array_equal(counts[:, :, 0], C)


@pytest.mark.parametrize("chunk", [(192, 64), (150, 37)])
def test_block_sparse_attention_is_sdpa_with_the_block_mask(chunk):
    w = small(24, G=2, Hkv=2, d=16, prefix=(128, 320), chunk=chunk, p=0.25)
    plans, counts = oracle.block_plans(w.masks, w.prefix_blocks, w.chunk_blocks, w.nkvb_max)
    O, L = oracle.block_sparse_attention(w.q, w.k_pages, w.v_pages, w.page_map, plans, counts, w.cu_q,
                                         w.prefix_len, w.Hkv)

    def token_mask(b, h):   # each row's own mask row, written out per token
        P, Cn = int(w.prefix_len[b]), int(w.chunk_len[b])
        m = np.zeros((Cn, P + Cn), dtype=bool)
        for r in range(Cn):
            for kb in range((P + Cn + BLOCK - 1) // BLOCK):
                if w.masks[b, h, r // BLOCK, kb]:
                    m[r, kb * BLOCK:(kb + 1) * BLOCK] = True
        return m
    Os, Ls = sdpa_dense(w, token_mask)
    assert np.max(np.abs(O - Os)) < 1e-12
    assert np.max(np.abs(L - Ls)) < 1e-12
    S = np.array([(b, h, r) for b in range(w.B) for h in range(w.Hq) for r in range(0, int(w.chunk_len[b]), 7)])
    Or, Lr = oracle.block_sparse_rows(w.q, w.k_pages, w.v_pages, w.page_map, plans, counts, w.cu_q,
                                      w.prefix_len, w.Hkv, S)
    # one row at a time against blocks of 64 rows: the same definition up to BLAS summation order
    assert np.max(np.abs(Or - O[w.cu_q[S[:, 0]] + S[:, 2], S[:, 1]])) < 1e-13
    assert np.max(np.abs(Lr - L[S[:, 1], w.cu_q[S[:, 0]] + S[:, 2]])) < 1e-13


def test_block_sparse_equals_union_when_masks_are_shared_and_constant():
    def fn(rng, Hq, Hkv, qb0, nqb, nkvb):
        s = rng.random((Hkv, nkvb)) < 0.3
        s[:, 0] = True
        return np.broadcast_to(np.repeat(s, Hq // Hkv, axis=0)[:, None, :], (Hq, nqb, nkvb)).copy()
    w = small(25, G=4, Hkv=2, d=16, prefix=(256, 512), chunk=(128, 192), fn=fn)
    plans, counts = oracle.block_plans(w.masks, w.prefix_blocks, w.chunk_blocks, w.nkvb_max)
    O, L = oracle.block_sparse_attention(w.q, w.k_pages, w.v_pages, w.page_map, plans, counts, w.cu_q,
                                         w.prefix_len, w.Hkv)
    Ou, Lu = run_oracle(w)
    assert np.max(np.abs(O - Ou)) < 1e-12 and np.max(np.abs(L - Lu)) < 1e-12


# ---- fp8 KV dequantization -------------------------------------------------------------------------

def test_decode_e4m3_worked_values():
    dec = oracle.decode_e4m3(np.array([0x38, 0x40, 0x7E, 0x01, 0x08, 0x80, 0x00, 0x7F, 0xFF, 0xB8, 0x3C], np.uint8))
    assert dec[0] == 1.0 and dec[1] == 2.0 and dec[2] == 448.0
    assert dec[3] == 2.0 ** -9 and dec[4] == 2.0 ** -6
    assert dec[5] == 0.0 and np.signbit(dec[5]) and dec[6] == 0.0 and not np.signbit(dec[6])
    assert np.isnan(dec[7]) and np.isnan(dec[8])
    assert dec[9] == -1.0 and dec[10] == 1.5


def test_decode_e4m3_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    dec = oracle.decode_e4m3(codes)
    assert np.array_equal(np.isnan(dec), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(dec[ok], ref[ok]) and np.array_equal(np.signbit(dec[ok]), np.signbit(ref[ok]))


def test_dequant_e4m3_is_decode_times_scale():
    y = oracle.dequant_e4m3(np.array([0x38, 0x3C, 0xC0], np.uint8), 0.3)
    s = float(np.float32(0.3))   # the scale as the library receives it (a C float)
    assert y.tolist() == [s, 1.5 * s, -2.0 * s]
