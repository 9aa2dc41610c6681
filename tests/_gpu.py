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


def sample_rows(w, n, seed=0):
    """(b, h, r) samples: random rows plus the first/last rows of tiles and of each chunk."""
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
    while len(out) < n:
        b = int(rng.integers(0, w.B))
        C = int(w.chunk_len[b])
        if C:
            out.add((b, int(rng.integers(0, w.Hq)), int(rng.integers(0, C))))
    return np.array(sorted(out), dtype=np.int64)
