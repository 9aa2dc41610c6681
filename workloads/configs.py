"""Seeded generators for the benchmark and test workloads.

Shapes follow the five workloads this path is measured on (a LLaMA-3.1-8B attention layer:
32 query heads, 8 KV heads, head dim 128; 128K context; chunks of 2048 and 4096 tokens; plus a
tiny fp32 case).  The model and the accuracy benchmark behind the published CompactAttention
figures are not available, so every tensor here is synthetic:

* Q, K and V are i.i.d. N(0, 1).  For bf16 workloads the fp32 samples are rounded to the nearest
  bf16 (ties to even) and kept as float32 arrays whose values are exactly representable in bf16,
  so that a device upload in bf16 is lossless and the oracle sees the same numbers.
* K/V live in a paged pool ``[n_pages][Hkv][64][d]``.  Logical blocks map to a seeded random
  permutation of physical pages; the pool holds 25% spare pages, one of which (``poison_page``)
  backs every page-map entry past a sequence's end.
* Masks are ``uint8 [B][Hq][nqb_max][nkvb_max]`` with nonzero = selected, drawn only on causal
  (Q-block, KV-block) entries unless a test asks for noise outside that region.

Only random draws and layout happen here; no union, table or attention arithmetic.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass, field

import numpy as np

BLOCK = 64  # tokens per Q-block, per KV-block and per page


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


@dataclass
class Workload:
    name: str
    Hq: int
    Hkv: int
    d: int
    dtype: str                 # "f32" or "bf16"
    prefix_len: np.ndarray     # int32 [B], tokens, multiple of 64
    chunk_len: np.ndarray      # int32 [B], tokens (need not be a multiple of 64)
    q: np.ndarray              # float32 [Tq][Hq][d]
    k_pages: np.ndarray        # float32 [n_pages][Hkv][64][d]
    v_pages: np.ndarray        # float32 [n_pages][Hkv][64][d]
    page_map: np.ndarray       # int32 [B][nkvb_max]: logical KV block -> physical page
    masks: np.ndarray          # uint8 [B][Hq][nqb_max][nkvb_max]
    poison_page: int           # a spare page no logical block maps to
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.prefix_len.shape[0])

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.chunk_len)]).astype(np.int32)

    @property
    def prefix_blocks(self) -> np.ndarray:
        return (self.prefix_len // BLOCK).astype(np.int32)

    @property
    def chunk_blocks(self) -> np.ndarray:
        return ((self.chunk_len + BLOCK - 1) // BLOCK).astype(np.int32)

    @property
    def nqb_max(self) -> int:
        return int(self.masks.shape[2])

    @property
    def nkvb_max(self) -> int:
        return int(self.masks.shape[3])

    @property
    def n_pages(self) -> int:
        return int(self.k_pages.shape[0])

    @property
    def max_chunk_len(self) -> int:
        return int(self.chunk_len.max()) if self.B else 0

    def used_pages(self) -> np.ndarray:
        """Boolean [n_pages]: pages some logical block of some sequence maps to."""
        used = np.zeros(self.n_pages, dtype=bool)
        for b in range(self.B):
            nk = int((self.prefix_len[b] + self.chunk_len[b] + BLOCK - 1) // BLOCK)
            used[self.page_map[b, :nk]] = True
        return used


# ----------------------------------------------------------------------------------------------
# mask patterns (per sequence): each returns bool [Hq][nQB][nKVB] before the causal clip
# ----------------------------------------------------------------------------------------------

def _causal(qb0: int, nqb: int, nkvb: int) -> np.ndarray:
    qi = np.arange(nqb)[:, None]
    kb = np.arange(nkvb)[None, :]
    return kb <= qb0 + qi


def _force_sink_and_local(m: np.ndarray, qb0: int, local: int) -> None:
    """Set KV block 0 and the `local` blocks ending at each Q-block's own diagonal block."""
    nqb = m.shape[1]
    m[:, :, 0] = True
    for qi in range(nqb):
        lo = max(0, qb0 + qi - local + 1)
        m[:, qi, lo:qb0 + qi + 1] = True


def mask_bernoulli(rng, Hq, Hkv, qb0, nqb, nkvb, p, local):
    m = rng.random((Hq, nqb, nkvb)) < p
    _force_sink_and_local(m, qb0, local)
    return m


def mask_structured(rng, Hq, Hkv, qb0, nqb, nkvb, stripe_p=0.03, n_slash=3, bern_p=0.02, local=4):
    """Vertical stripes (one draw per head and KV block, applied to every Q-block), slash
    diagonals at random offsets, per-entry Bernoulli noise, sink block 0 and a local window."""
    stripes = rng.random((Hq, nkvb)) < stripe_p
    m = np.broadcast_to(stripes[:, None, :], (Hq, nqb, nkvb)).copy()
    offs = rng.integers(0, qb0 + 1, size=(Hq, n_slash))
    qi = np.arange(nqb)
    for h in range(Hq):
        for o in offs[h]:
            m[h, qi, qb0 + qi - o] = True
    if bern_p > 0:
        m |= rng.random((Hq, nqb, nkvb)) < bern_p
    _force_sink_and_local(m, qb0, local)
    return m


def mask_stripes(rng, Hq, Hkv, qb0, nqb, nkvb, p, shared_per_group):
    """Vertical stripes of density p; one stripe set per KV group (shared by its query heads)
    or one per query head; sink block 0 and each Q-block's diagonal block forced on."""
    G = Hq // Hkv
    if shared_per_group:
        s = rng.random((Hkv, nkvb)) < p
        s = np.repeat(s, G, axis=0)
    else:
        s = rng.random((Hq, nkvb)) < p
    m = np.broadcast_to(s[:, None, :], (Hq, nqb, nkvb)).copy()
    _force_sink_and_local(m, qb0, 1)
    return m


def mask_all(rng, Hq, Hkv, qb0, nqb, nkvb, value):
    return np.full((Hq, nqb, nkvb), bool(value))


# ----------------------------------------------------------------------------------------------
# generic builder
# ----------------------------------------------------------------------------------------------

def _normal(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def make_workload(name, prefix_len, chunk_len, Hq, Hkv, d, dtype, mask_fn, seed,
                  pool_factor=1.25, noncausal_noise=0.0, mask_values=False, kv=None, q=None):
    """Build one seeded workload.

    mask_fn(rng, Hq, Hkv, qb0, nqb, nkvb) -> bool [Hq][nqb][nkvb] is called per sequence; entries
    outside the causal region are cleared, then (for tests of the clip) optionally refilled with
    Bernoulli(noncausal_noise) noise, as is the padding past each sequence's own extent.
    mask_values=True stores random nonzero byte values instead of 1 for selected entries.
    kv=(k_pages, v_pages, page_map_rows) reuses an existing pool; q reuses a Q array.
    """
    prefix_len = np.asarray(prefix_len, dtype=np.int32)
    chunk_len = np.asarray(chunk_len, dtype=np.int32)
    if np.any(prefix_len % BLOCK) or np.any(prefix_len < 0) or np.any(chunk_len < 0):
        raise ValueError("prefix lengths must be non-negative multiples of 64")
    B = prefix_len.shape[0]
    ss = np.random.SeedSequence(seed)
    rq, rk, rv, rm, rp = [np.random.default_rng(s) for s in ss.spawn(5)]
    qb0 = prefix_len // BLOCK
    nqb = (chunk_len + BLOCK - 1) // BLOCK   # a ragged chunk ends in a partial query block
    nkvb = qb0 + nqb
    nqb_max = int(nqb.max()) if B else 0
    nkvb_max = int(nkvb.max()) if B else 0
    Tq = int(chunk_len.sum())

    masks = np.zeros((B, Hq, nqb_max, nkvb_max), dtype=np.uint8)
    for b in range(B):
        m = mask_fn(rm, Hq, Hkv, int(qb0[b]), int(nqb[b]), int(nkvb[b]))
        m = m & _causal(int(qb0[b]), int(nqb[b]), int(nkvb[b]))[None]
        masks[b, :, :nqb[b], :nkvb[b]] = m
    if noncausal_noise > 0:
        noise = rm.random(masks.shape) < noncausal_noise
        for b in range(B):
            inside = np.zeros((nqb_max, nkvb_max), dtype=bool)
            inside[:nqb[b], :nkvb[b]] = _causal(int(qb0[b]), int(nqb[b]), int(nkvb[b]))
            masks[b] |= (noise[b] & ~inside[None]).astype(np.uint8)
    if mask_values:
        vals = rm.integers(1, 256, size=masks.shape, dtype=np.uint8)
        masks = np.where(masks != 0, vals, np.uint8(0)).astype(np.uint8)

    if kv is None:
        total = int(nkvb.sum())
        n_pages = max(total + 1, int(math.ceil(total * pool_factor)))
        perm = rp.permutation(n_pages).astype(np.int32)
        page_map = np.full((B, max(nkvb_max, 1)), perm[total], dtype=np.int32)
        off = 0
        for b in range(B):
            page_map[b, :nkvb[b]] = perm[off:off + nkvb[b]]
            off += int(nkvb[b])
        poison = int(perm[total])
        k_pages = _normal(rk, (n_pages, Hkv, BLOCK, d), dtype)
        v_pages = _normal(rv, (n_pages, Hkv, BLOCK, d), dtype)
    else:
        k_pages, v_pages, page_map, poison = kv
    if q is None:
        q = _normal(rq, (Tq, Hq, d), dtype)
    return Workload(name, Hq, Hkv, d, dtype, prefix_len, chunk_len, q, k_pages, v_pages,
                    page_map, masks, poison, meta={"seed": seed})


# ----------------------------------------------------------------------------------------------
# the named workloads
# ----------------------------------------------------------------------------------------------

CONFIG_NAMES = (
    "c1_tiny_f32",              # 1K context, fp32, Hq 8 / Hkv 2, d 64, chunk 256
    "c2_32k_bf16",              # 30720 prefix + 2048 chunk, bf16 LLaMA-3.1-8B layer shape
    "c3_128k_last_chunk",       # 129024 prefix + 2048 chunk, structured masks (headline)
    "c4_128k_chunked",          # chunk k of a 131072-token sequence (64 chunks of 2048)
    "c5a_varlen_shared",        # 4 sequences (8K/32K/64K/128K), last 4096, group-shared stripes
    "c5b_varlen_independent",   # same, independent stripes per head
)

SEEDS = {"c1_tiny_f32": 1001, "c2_32k_bf16": 1002, "c3_128k_last_chunk": 1003,
         "c4_128k_chunked": 1004, "c5a_varlen_shared": 1005, "c5b_varlen_independent": 1006,
         "c3s_128k_one_group": 1007, "c3d_128k_no_noise": 1003, "c3g7_128k_gqa7": 1008}

# One KV group's share of the 128K last-chunk workload: what each of 8 GPUs would hold if the
# layer's 8 KV groups were split across them (4 query heads, 1 KV head); 32 query tiles.
SHARD_NAMES = ("c3s_128k_one_group",)

# A diagnostic, never a replacement for the headline workload: the 128K last chunk with the same
# seed and generator but without the per-entry Bernoulli(0.02) term, so its stripes, slashes, sink
# and local window are exactly the headline's and the group unions stay sparse (about a quarter
# of the blocks) instead of near-dense.
DIAG_NAMES = ("c3d_128k_no_noise",)

# A parity case for a group size that is not a power of two: the 128K last chunk with 28 query
# heads over 4 KV heads (G = 7, a grouping some GQA models use), the headline's mask generator.
GQA_NAMES = ("c3g7_128k_gqa7",)

C4_SEQ = 131072
C4_CHUNK = 2048


@functools.lru_cache(maxsize=2)
def _c4_pool(seed: int):
    """Paged K/V of the whole 131072-token sequence, shared by all 64 chunks."""
    ss = np.random.SeedSequence(seed)
    rk, rv, rp = [np.random.default_rng(s) for s in ss.spawn(3)]
    total = C4_SEQ // BLOCK
    n_pages = int(math.ceil(total * 1.25))
    perm = rp.permutation(n_pages).astype(np.int32)
    k = _normal(rk, (n_pages, 8, BLOCK, 128), "bf16")
    v = _normal(rv, (n_pages, 8, BLOCK, 128), "bf16")
    return k, v, perm[:total].copy(), int(perm[total])


def chunked_sequence_chunk(k: int, dense: bool = False, seed: int | None = None) -> Workload:
    """Chunk k (0..63) of the 131072-token sequence: prefix 2048*k, chunk 2048, its own
    seeded structured mask (or all-ones when dense=True) over its causal prefix."""
    base = SEEDS["c4_128k_chunked"] if seed is None else seed
    kp, vp, blocks, poison = _c4_pool(base)
    P = C4_CHUNK * k
    nk = (P + C4_CHUNK) // BLOCK
    page_map = blocks[None, :nk].copy()
    fn = (lambda rng, *a: mask_all(rng, *a, value=1)) if dense else mask_structured
    w = make_workload(f"c4_128k_chunked[{k}]" + ("_dense" if dense else ""), [P], [C4_CHUNK],
                      32, 8, 128, "bf16", fn, base + 1 + k, kv=(kp, vp, page_map, poison))
    return w


def pack_mask_bits(masks: np.ndarray) -> np.ndarray:
    """Byte masks [B][Hq][nqb][nkvb] (nonzero = selected) as bit-packed uint64 words
    [B][Hq][nqb][ceil(nkvb/64)]: block kb is bit kb % 64 of word kb // 64 (an input encoding)."""
    B, Hq, nqb, nkvb = masks.shape
    words = (nkvb + 63) // 64
    padded = np.zeros((B, Hq, nqb, words * 64), dtype=np.uint8)
    padded[..., :nkvb] = masks != 0
    return np.packbits(padded.reshape(B, Hq, nqb, words, 64), axis=-1, bitorder="little").view(np.uint64)[..., 0]


def chunked_sequence_batch(dense: bool = False, seed: int | None = None, n_chunks: int = 64) -> Workload:
    """The first n_chunks chunks of the 131072-token sequence as one varlen batch: sequence k of
    the batch is chunk k (prefix 2048*k, chunk 2048) with the Q, mask and page map of
    chunked_sequence_chunk(k), all over the one shared paged pool."""
    parts = [chunked_sequence_chunk(k, dense=dense, seed=seed) for k in range(n_chunks)]
    last = parts[-1]
    nqb = C4_CHUNK // BLOCK
    nkvb = max(p.nkvb_max for p in parts)
    masks = np.zeros((n_chunks, last.Hq, nqb, nkvb), dtype=np.uint8)
    page_map = np.full((n_chunks, nkvb), last.poison_page, dtype=np.int32)
    for k, p in enumerate(parts):
        masks[k, :, :, :p.nkvb_max] = p.masks[0]
        page_map[k, :p.page_map.shape[1]] = p.page_map[0]
    return Workload("c4_128k_chunked_batch" + ("_dense" if dense else ""), last.Hq, last.Hkv, last.d, last.dtype,
                    np.array([p.prefix_len[0] for p in parts], dtype=np.int32),
                    np.array([p.chunk_len[0] for p in parts], dtype=np.int32),
                    np.concatenate([p.q for p in parts], axis=0), last.k_pages, last.v_pages, page_map, masks,
                    last.poison_page, meta={"seed": last.meta.get("seed"), "chunks": n_chunks})


def make_config(name: str, dense: bool = False, chunk: int = 63, seed: int | None = None) -> Workload:
    """One of the named workloads; dense=True swaps every mask for all-ones (the dense run)."""
    s = SEEDS[name] if seed is None else seed
    ones = lambda rng, *a: mask_all(rng, *a, value=1)  # noqa: E731
    if name == "c1_tiny_f32":
        fn = ones if dense else (lambda rng, *a: mask_bernoulli(rng, *a, p=0.3, local=1))
        return make_workload(name, [768], [256], 8, 2, 64, "f32", fn, s)
    if name == "c2_32k_bf16":
        fn = ones if dense else (lambda rng, *a: mask_bernoulli(rng, *a, p=0.1, local=4))
        return make_workload(name, [30720], [2048], 32, 8, 128, "bf16", fn, s)
    if name == "c3_128k_last_chunk":
        fn = ones if dense else mask_structured
        return make_workload(name, [129024], [2048], 32, 8, 128, "bf16", fn, s)
    if name == "c4_128k_chunked":
        return chunked_sequence_chunk(chunk, dense=dense, seed=seed)
    if name == "c3d_128k_no_noise":
        fn = ones if dense else (lambda rng, *a: mask_structured(rng, *a, bern_p=0.0))
        return make_workload(name, [129024], [2048], 32, 8, 128, "bf16", fn, s)
    if name == "c3g7_128k_gqa7":
        fn = ones if dense else mask_structured
        return make_workload(name, [129024], [2048], 28, 4, 128, "bf16", fn, s)
    if name == "c3s_128k_one_group":
        fn = ones if dense else mask_structured
        return make_workload(name, [129024], [2048], 4, 1, 128, "bf16", fn, s)
    if name in ("c5a_varlen_shared", "c5b_varlen_independent"):
        shared = name == "c5a_varlen_shared"
        L = np.array([8192, 32768, 65536, 131072])
        C = np.full(4, 4096)
        fn = ones if dense else (lambda rng, *a: mask_stripes(rng, *a, p=0.1, shared_per_group=shared))
        return make_workload(name, L - C, C, 32, 8, 128, "bf16", fn, s)
    raise KeyError(name)
