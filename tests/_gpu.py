"""Helpers shared by the GPU tests: upload a seeded workload, run the library, compare."""
import numpy as np
import torch

import sparse_attention_long_reduce_amd as cpa

BF16_MAX, BF16_MEAN, BF16_RELL2 = 2e-2, 2e-3, 2e-2   # bf16 inputs (rel-L2 is an extra guard)
F32_MAX = 1e-4                                       # fp32 inputs


def tdtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def upload(w, dev="cuda", k_pages=None, v_pages=None, page_map=None):
    dt = tdtype(w)
    kp = w.k_pages if k_pages is None else k_pages
    vp = w.v_pages if v_pages is None else v_pages
    pm = w.page_map if page_map is None else page_map
    return {
        "masks": torch.from_numpy(np.ascontiguousarray(w.masks)).to(dev),
        "pb": torch.from_numpy(w.prefix_blocks).to(dev),
        "cb": torch.from_numpy(w.chunk_blocks).to(dev),
        "q": torch.from_numpy(w.q).to(dev).to(dt),
        "kp": torch.from_numpy(kp).to(dev).to(dt),
        "vp": torch.from_numpy(vp).to(dev).to(dt),
        "pm": torch.from_numpy(np.ascontiguousarray(pm)).to(dev),
        "cu": torch.from_numpy(w.cu_q).to(dev),
        "pl": torch.from_numpy(w.prefix_len).to(dev),
    }


def gpu_tables(dv, w, cap=None):
    return cpa.build_block_tables(dv["masks"], dv["pb"], dv["cb"], w.Hkv, table_cap=cap)


def gpu_prefill(dv, w, tables, counts, kp=None, vp=None):
    return cpa.chunked_prefill(dv["q"], dv["kp"] if kp is None else kp, dv["vp"] if vp is None else vp,
                               dv["pm"], tables, counts, dv["cu"], dv["pl"], w.max_chunk_len,
                               return_lse=True)


def compare(w, o_gpu, O_ref, what=""):
    """Element-wise comparison at the tolerance for the workload's dtype; returns the errors."""
    o = o_gpu.float().cpu().numpy().astype(np.float64) if isinstance(o_gpu, torch.Tensor) else o_gpu
    err = np.abs(o - O_ref)
    mx, mean = float(err.max()), float(err.mean())
    rel = float(np.linalg.norm(o - O_ref) / max(np.linalg.norm(O_ref), 1e-300))
    if w.dtype == "bf16":
        assert mx <= BF16_MAX and mean <= BF16_MEAN and rel <= BF16_RELL2, \
            f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}"
    else:
        assert mx <= F32_MAX, f"{what}: max-abs {mx:.3e}"
    return mx, mean, rel


def sample_rows(w, n, seed=0, per_tile=2):
    """(b, h, r) samples that reach every tile of the prefill: for every sequence b, KV group g
    and query block qi, `per_tile` rows of that block (one in each 32-row half, the halves two
    different waves compute) at random heads of g; the first/last rows of tiles and of each
    chunk; and random rows until there are at least n beyond the per-tile ones."""
    rng = np.random.default_rng(seed)
    out = set()
    for b in range(w.B):
        C = int(w.chunk_len[b])
        if C == 0:
            continue
        for h in (0, w.Hq - 1, int(rng.integers(0, w.Hq))):
            for r in (0, 31, 32, 63, 64, C - 64, C - 33, C - 1):
                if 0 <= r < C:
                    out.add((b, h, r))
        for g in range(w.Hkv):
            for qi in range((C + 63) // 64):
                for k in range(per_tile):
                    lo = 64 * qi + 32 * (k % 2)
                    hi = min(C, lo + 32)
                    if lo >= C:
                        lo, hi = 64 * qi, min(C, 64 * qi + 64)
                    out.add((b, g * w.G + int(rng.integers(0, w.G)), int(rng.integers(lo, hi))))
    n_tile = len(out)
    while len(out) < n_tile + n:
        b = int(rng.integers(0, w.B))
        C = int(w.chunk_len[b])
        if C:
            out.add((b, int(rng.integers(0, w.Hq)), int(rng.integers(0, C))))
    return np.array(sorted(out), dtype=np.int64)


def tiles_reached(w, S):
    """Number of (sequence, KV group, query block) tiles that the samples S reach, and the total."""
    seen = {(int(b), int(h) // w.G, int(r) // 64) for b, h, r in S}
    total = sum(w.Hkv * ((int(c) + 63) // 64) for c in w.chunk_len)
    return len(seen), total


def oracle_full(w, T, C, q=None, k_pages=None, v_pages=None, workers=None):
    """The oracle's O [Tq][Hq][d] and LSE [Hq][Tq] for every row, computed one (sequence, KV
    group, row range) at a time in a thread pool: each piece is oracle.paged_attention on that
    sequence's rows and that group's heads and pages (groups and rows are independent by the
    definition), with BLAS kept to one thread per piece."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_limits
    q = w.q if q is None else q
    kp = w.k_pages if k_pages is None else k_pages
    vp = w.v_pages if v_pages is None else v_pages
    Tq, Hq, d = q.shape
    G = w.G
    O = np.zeros((Tq, Hq, d), dtype=np.float64)
    LSE = np.full((Hq, Tq), -np.inf, dtype=np.float64)
    workers = workers or min(16, os.cpu_count() or 1)
    pieces = []
    n_bg = max(1, sum(1 for b in range(w.B) if w.chunk_len[b] > 0) * w.Hkv)
    for b in range(w.B):
        q0, q1 = int(w.cu_q[b]), int(w.cu_q[b + 1])
        if q1 == q0:
            continue
        n_split = max(1, min(-(-workers // n_bg), (q1 - q0) // 64))
        step = -(-(q1 - q0) // (64 * n_split)) * 64
        for g in range(w.Hkv):
            for r0 in range(0, q1 - q0, step):
                pieces.append((b, g, r0, min(q1 - q0, r0 + step)))

    def run(piece):
        b, g, r0, r1 = piece
        q0 = int(w.cu_q[b])
        o, lse = oracle.paged_attention(
            q[q0 + r0:q0 + r1, g * G:(g + 1) * G], kp[:, g:g + 1], vp[:, g:g + 1], w.page_map[b:b + 1],
            T[b:b + 1, g:g + 1], C[b:b + 1, g:g + 1], np.array([0, r1 - r0], dtype=np.int64),
            np.array([int(w.prefix_len[b]) + r0], dtype=np.int64), 1)
        O[q0 + r0:q0 + r1, g * G:(g + 1) * G] = o
        LSE[g * G:(g + 1) * G, q0 + r0:q0 + r1] = lse

    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        list(ex.map(run, pieces))
    return O, LSE


def error_stats(o, O_ref):
    """max-abs, mean-abs and rel-L2 of o (GPU, any float dtype) against the fp64 oracle."""
    o = o.float().cpu().numpy().astype(np.float64) if isinstance(o, torch.Tensor) else np.asarray(o, np.float64)
    err = np.abs(o - O_ref)
    return {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
            "rel_l2": float(np.linalg.norm(o - O_ref) / max(np.linalg.norm(O_ref), 1e-300)),
            "ref_rms": float(np.sqrt(np.mean(O_ref ** 2))), "elements": int(err.size)}


def report(name, stats):
    """Print one parity line and, when CPA_PARITY_REPORT names a file, append it there as JSON."""
    import json
    import os
    line = {"case": name, **stats}
    print(f"[parity] {json.dumps(line)}", flush=True)
    path = os.environ.get("CPA_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")
