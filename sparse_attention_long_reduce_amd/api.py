"""Python binding of the C ABI: argument marshalling only.

torch supplies device memory and the current HIP stream; every step of the path runs in the
library's HIP kernels.  Names and semantics follow include/cpa.h.
"""
import math

import torch

from ._lib import CpaError, load

BLOCK = 64
F32, BF16, FP8_E4M3 = 0, 1, 2
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}
_KV_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3}


def _stream(stream, dev):
    """The HIP stream handle to launch on: `stream` (which must belong to dev) or dev's current one."""
    s = torch.cuda.current_stream(dev) if stream is None else stream
    if s.device != dev:
        raise ValueError(f"the stream belongs to {s.device}, the tensors to {dev}")
    return s.cuda_stream


def _on(dev, **tensors):
    """Check that every given tensor (None skipped) is a CUDA tensor on dev; returns dev."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not (isinstance(t, torch.Tensor) and t.is_cuda):
            raise TypeError(f"{name} must be a CUDA tensor")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the call's other tensors on {dev}")
    return dev


def _cuda_device(t, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda):
        raise TypeError(f"{name} must be a CUDA tensor")
    return t.device


def _dev_i32(x, name):
    if not (isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == torch.int32 and x.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous int32 CUDA tensor")
    return x


def _i32(x, name):
    """Dtype and layout of an int32 index tensor (its device is checked with the others)."""
    if not (isinstance(x, torch.Tensor) and x.dtype == torch.int32 and x.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    return x


def _chunk_cap(cu_q, max_chunk_len, stream, dev):
    """max_chunk_len as given, or (None) the longest chunk cu_q[b+1] - cu_q[b], read from the
    device on the call's stream (`stream`, else dev's current one), after the work queued there:
    one synchronisation with that stream, so a call under graph capture must pass it."""
    if max_chunk_len is not None:
        return int(max_chunk_len)
    if cu_q.numel() < 2:
        return 0
    s = torch.cuda.current_stream(dev) if stream is None else stream
    if s.device != dev:
        raise ValueError(f"the stream belongs to {s.device}, the tensors to {dev}")
    with torch.cuda.device(dev), torch.cuda.stream(s):
        return max(int((cu_q[1:] - cu_q[:-1]).max().item()), 0)


def _scale(sm_scale):
    """The softmax scale for the C ABI: 0 (the library then takes 1/sqrt(d)) for None."""
    return 0.0 if sm_scale is None else float(sm_scale)


def _out_buffers(out, lse, return_lse, q, dev):
    """Validate caller-given o / lse (contiguous, q's shape and dtype / float32 [Tq][Hq]) or
    allocate them."""
    Tq, Hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty_like(q)
    elif not (out.is_contiguous() and out.shape == q.shape and out.dtype == q.dtype):
        raise ValueError("out must be a contiguous tensor of q's shape and dtype")
    if lse is None and return_lse:
        lse = torch.empty((Tq, Hq), dtype=torch.float32, device=dev)
    elif lse is not None and not (lse.is_contiguous() and tuple(lse.shape) == (Tq, Hq) and lse.dtype == torch.float32):
        raise ValueError("lse must be a contiguous float32 [Tq][Hq] tensor")
    _on(dev, out=out, lse=lse)
    return out, lse


def _ptr(x):
    return None if x is None else x.data_ptr()


def build_block_tables(masks, prefix_blocks, chunk_blocks, Hkv, table_cap=None, tables=None,
                       counts=None, stream=None):
    """masks uint8 [B][Hq][nqb_max][nkvb_max] (CUDA) -> (tables int32 [B][Hkv][cap], counts int32 [B][Hkv]).

    prefix_blocks / chunk_blocks are int32 CUDA tensors [B].  Output tensors may be passed in.
    """
    if not (masks.is_cuda and masks.dtype == torch.uint8 and masks.is_contiguous() and masks.dim() == 4):
        raise TypeError("masks must be a contiguous 4-D uint8 CUDA tensor")
    dev = masks.device
    B, Hq, nqb_max, nkvb_max = masks.shape
    _dev_i32(prefix_blocks, "prefix_blocks")
    _dev_i32(chunk_blocks, "chunk_blocks")
    cap = nkvb_max if table_cap is None else int(table_cap)
    if tables is None:
        tables = torch.empty((B, Hkv, cap), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    _dev_i32(tables, "tables")
    _dev_i32(counts, "counts")
    if tables.numel() != B * Hkv * cap or counts.numel() != B * Hkv:
        raise ValueError("tables/counts have the wrong size")
    _on(dev, prefix_blocks=prefix_blocks, chunk_blocks=chunk_blocks, tables=tables, counts=counts)
    with torch.cuda.device(dev):
        st = load().cpa_build_block_tables(_ptr(masks), B, Hq, Hkv, nqb_max, nkvb_max,
                                           _ptr(prefix_blocks), _ptr(chunk_blocks), _ptr(tables), cap,
                                           _ptr(counts), _stream(stream, dev))
    if st != 0:
        raise CpaError(st, "cpa_build_block_tables")
    return tables, counts


def build_block_tables_bits(mask_bits, nkvb_max, prefix_blocks, chunk_blocks, Hkv, table_cap=None, tables=None,
                            counts=None, stream=None):
    """Bit-packed masks int64 [B][Hq][nqb_max][words] (CUDA; bit kb % 64 of word kb / 64 = block
    kb selected, the words' bits taken as unsigned) -> (tables, counts) as build_block_tables."""
    if not (mask_bits.is_cuda and mask_bits.dtype in (torch.int64, torch.uint64) and mask_bits.is_contiguous()
            and mask_bits.dim() == 4):
        raise TypeError("mask_bits must be a contiguous 4-D int64 CUDA tensor")
    dev = mask_bits.device
    B, Hq, nqb_max, words = mask_bits.shape
    _dev_i32(prefix_blocks, "prefix_blocks")
    _dev_i32(chunk_blocks, "chunk_blocks")
    cap = int(nkvb_max) if table_cap is None else int(table_cap)
    if tables is None:
        tables = torch.empty((B, Hkv, cap), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    _dev_i32(tables, "tables")
    _dev_i32(counts, "counts")
    if tables.numel() != B * Hkv * cap or counts.numel() != B * Hkv:
        raise ValueError("tables/counts have the wrong size")
    _on(dev, prefix_blocks=prefix_blocks, chunk_blocks=chunk_blocks, tables=tables, counts=counts)
    with torch.cuda.device(dev):
        st = load().cpa_build_block_tables_bits(_ptr(mask_bits), B, Hq, Hkv, nqb_max, int(nkvb_max), words,
                                                _ptr(prefix_blocks), _ptr(chunk_blocks), _ptr(tables), cap,
                                                _ptr(counts), _stream(stream, dev))
    if st != 0:
        raise CpaError(st, "cpa_build_block_tables_bits")
    return tables, counts


def build_block_plans(masks, prefix_blocks, chunk_blocks, plan_cap=None, plans=None, plan_counts=None,
                      stream=None):
    """masks uint8 [B][Hq][nqb_max][nkvb_max] (CUDA) -> per-(head, query block) plans of the
    direct block-sparse baseline: (plans int32 [B][Hq][nqb_max][cap], counts int32 [B][Hq][nqb_max])."""
    if not (masks.is_cuda and masks.dtype == torch.uint8 and masks.is_contiguous() and masks.dim() == 4):
        raise TypeError("masks must be a contiguous 4-D uint8 CUDA tensor")
    dev = masks.device
    B, Hq, nqb_max, nkvb_max = masks.shape
    _dev_i32(prefix_blocks, "prefix_blocks")
    _dev_i32(chunk_blocks, "chunk_blocks")
    cap = nkvb_max if plan_cap is None else int(plan_cap)
    if plans is None:
        plans = torch.empty((B, Hq, nqb_max, cap), dtype=torch.int32, device=dev)
    if plan_counts is None:
        plan_counts = torch.empty((B, Hq, nqb_max), dtype=torch.int32, device=dev)
    _dev_i32(plans, "plans")
    _dev_i32(plan_counts, "plan_counts")
    if plans.numel() != B * Hq * nqb_max * cap or plan_counts.numel() != B * Hq * nqb_max:
        raise ValueError("plans/plan_counts have the wrong size")
    _on(dev, prefix_blocks=prefix_blocks, chunk_blocks=chunk_blocks, plans=plans, plan_counts=plan_counts)
    with torch.cuda.device(dev):
        st = load().cpa_build_block_plans(_ptr(masks), B, Hq, nqb_max, nkvb_max, _ptr(prefix_blocks),
                                          _ptr(chunk_blocks), _ptr(plans), cap, _ptr(plan_counts),
                                          _stream(stream, dev))
    if st != 0:
        raise CpaError(st, "cpa_build_block_plans")
    return plans, plan_counts


def chunked_prefill_direct(q, k_pages, v_pages, page_map, plans, plan_counts, cu_q, prefix_len, max_chunk_len=None,
                           sm_scale=None, out=None, lse=None, return_lse=False, stream=None):
    """Direct block-sparse baseline: each (head, query block) over its own plan.  q bf16
    [Tq][Hq][d]; k_pages [n_pages][Hkv][64][d]; v_pages dim-major [n_pages][Hkv][d][64] (strided
    views allowed as in chunked_prefill); plans / plan_counts from build_block_plans;
    max_chunk_len as in chunked_prefill."""
    if q.dtype != torch.bfloat16 or k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("the direct baseline runs bf16 q, k_pages and v_pages")
    if q.dim() != 3 or not q.is_contiguous():
        raise TypeError("q must be a contiguous [Tq][Hq][d] tensor")
    Tq, Hq, d = q.shape
    if k_pages.dim() != 4 or k_pages.shape[2] != BLOCK or k_pages.shape[3] != d or k_pages.stride(3) != 1:
        raise ValueError("k_pages must be [n_pages][Hkv][64][d] with d contiguous")
    n_pages, Hkv = k_pages.shape[0], k_pages.shape[1]
    if v_pages.dim() != 4 or tuple(v_pages.shape) != (n_pages, Hkv, d, BLOCK) or v_pages.stride(3) != 1:
        raise ValueError("v_pages must be dim-major [n_pages][Hkv][d][64] with the token dimension contiguous")
    for t, nm in ((page_map, "page_map"), (plans, "plans"), (plan_counts, "plan_counts"), (cu_q, "cu_q"),
                  (prefix_len, "prefix_len")):
        _i32(t, nm)
    B = prefix_len.numel()
    if plans.dim() != 4 or plans.shape[0] != B or plans.shape[1] != Hq:
        raise ValueError("plans must be [B][Hq][nqb_max][cap]")
    nqb_max, cap = plans.shape[2], plans.shape[3]
    if tuple(plan_counts.shape) != (B, Hq, nqb_max):
        raise ValueError("plan_counts must be [B][Hq][nqb_max], matching plans")
    if cu_q.numel() != B + 1 or page_map.dim() != 2 or page_map.shape[0] != B:
        raise ValueError("inconsistent B across cu_q / prefix_len / page_map")
    dev = _on(_cuda_device(q, "q"), k_pages=k_pages, v_pages=v_pages, page_map=page_map, plans=plans,
              plan_counts=plan_counts, cu_q=cu_q, prefix_len=prefix_len)
    max_chunk_len = _chunk_cap(cu_q, max_chunk_len, stream, dev)
    out, lse = _out_buffers(out, lse, return_lse, q, dev)
    with torch.cuda.device(dev):
        st = load().cpa_chunked_prefill_direct(
            _ptr(q), BF16, _ptr(k_pages), k_pages.stride(0), k_pages.stride(1), k_pages.stride(2), _ptr(v_pages),
            v_pages.stride(0), v_pages.stride(1), v_pages.stride(2), n_pages, _ptr(page_map), page_map.shape[1],
            _ptr(plans), cap, _ptr(plan_counts), nqb_max, _ptr(cu_q), _ptr(prefix_len), B, Hq, Hkv, d,
            int(max_chunk_len), _scale(sm_scale), _ptr(out), _ptr(lse), _stream(stream, dev))
    if st != 0:
        raise CpaError(st, "cpa_chunked_prefill_direct")
    return out, lse


def plan_flops(plans, plan_counts, prefix_len, chunk_len, d):
    """FLOPs of the direct baseline, 4*d per causally visible (query, key) pair of every
    (head, query block) plan, from host copies (numpy) of the plans."""
    import numpy as np
    total = 0
    B, Hq, nqb_max, _ = plans.shape
    for b in range(B):
        P, C = int(prefix_len[b]), int(chunk_len[b])
        for qi in range((C + BLOCK - 1) // BLOCK):
            r = np.arange(BLOCK * qi, min(C, BLOCK * qi + BLOCK), dtype=np.int64)
            for h in range(Hq):
                ids = np.asarray(plans[b, h, qi, :plan_counts[b, h, qi]], dtype=np.int64)
                full = ids[ids * BLOCK + BLOCK - 1 <= P + BLOCK * qi]   # blocks wholly before the query block
                pairs = int(full.size) * BLOCK * r.size
                for kb in ids[ids * BLOCK + BLOCK - 1 > P + BLOCK * qi]:
                    pairs += int(np.clip(P + r - kb * BLOCK + 1, 0, BLOCK).sum())
                total += pairs
    return 4 * d * total


PAIRS_PER_TILE = 4   # (query block, head) pairs per prefill workgroup


def prefill_tiles(B, Hq, Hkv, max_chunk_len):
    """Workgroups cpa_chunked_prefill launches without split-KV: per KV group, its (query block,
    head) pairs in tiles of four consecutive ones (pairs numbered query block * G + head)."""
    G = Hq // Hkv
    nqb = -(-int(max_chunk_len) // BLOCK)
    return B * Hkv * -(-(nqb * G) // PAIRS_PER_TILE)


def plan_split_pages(B, Hq, Hkv, max_chunk_len, table_cap, n_cus, max_splits=16):
    """Pages per split-KV range so that the tiles times their ranges cover every CU once when the
    tiles alone would leave CUs idle; 0 (no split) when there are at least as many tiles as CUs."""
    tiles = prefill_tiles(B, Hq, Hkv, max_chunk_len)
    if tiles == 0 or tiles >= n_cus or table_cap <= 1:
        return 0
    splits = min(max_splits, -(-n_cus // tiles), table_cap)
    return -(-table_cap // splits) if splits > 1 else 0


def split_workspace_bytes(total_q, Hq, d, table_cap, split_pages):
    return int(load().cpa_split_workspace_bytes(int(total_q), int(Hq), int(d), int(table_cap), int(split_pages)))


def chunked_prefill(q, k_pages, v_pages, page_map, tables, counts, cu_q, prefix_len, max_chunk_len=None,
                    sm_scale=None, out=None, lse=None, return_lse=False, stream=None, split_pages=0,
                    workspace=None, v_layout="token", k_scale=1.0, v_scale=1.0):
    """Attention of each sequence's chunk over its group's table blocks, K/V read in place.

    q [Tq][Hq][d]; k_pages [n_pages][Hkv][64][d] (or any strided view with d contiguous);
    v_pages the same (v_layout "token") or dim-major [n_pages][Hkv][d][64] (v_layout "dim", any
    strided view with the token dimension contiguous); page_map int32 [B][stride]; tables int32
    [B][Hkv][cap]; counts int32 [B][Hkv]; cu_q int32 [B+1]; prefix_len int32 [B]; max_chunk_len
    a host int at least the longest chunk, or None to read it from cu_q (one synchronisation
    with the device).  sm_scale: the softmax scale, None or 0 for 1/sqrt(d).  Returns
    (o, lse-or-None).

    split_pages > 0 runs split-KV (cpa_chunked_prefill_split) with ranges of that many pages;
    the workspace (a CUDA uint8 tensor of split_workspace_bytes(...) bytes) is allocated here
    when not given.  split_pages="auto" picks the range length with plan_split_pages for the
    device's compute units: a split when the call has fewer tiles than CUs and the split kernel
    takes the pools (bf16 q, bf16 or fp8 pools, row strides up to 2^24 elements), else none.
    v_layout "dim" calls cpa_chunked_prefill_vt.  float8_e4m3fn pools with a bf16 q call
    cpa_chunked_prefill_fp8kv (split or not) with the dequantization scales k_scale / v_scale.
    """
    auto = isinstance(split_pages, str)
    if auto and split_pages != "auto":
        raise ValueError('split_pages must be an int or "auto"')
    fp8 = k_pages.dtype == torch.float8_e4m3fn
    if fp8:
        if q.dtype != torch.bfloat16 or v_pages.dtype != k_pages.dtype:
            raise TypeError("fp8 pools need float8_e4m3fn k_pages and v_pages and a bfloat16 q")
    elif q.dtype not in _DTYPES or k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("q, k_pages and v_pages must share dtype float32 or bfloat16")
    if q.dim() != 3 or not q.is_contiguous():
        raise TypeError("q must be a contiguous [Tq][Hq][d] tensor")
    Tq, Hq, d = q.shape
    if k_pages.dim() != 4 or k_pages.shape[2] != BLOCK or k_pages.shape[3] != d:
        raise ValueError("k_pages must be [n_pages][Hkv][64][d]")
    if v_layout == "token":
        if v_pages.shape != k_pages.shape or v_pages.stride() != k_pages.stride():
            raise ValueError("v_pages must match k_pages in shape and strides")
    elif v_layout == "dim":
        n_p, h_p = k_pages.shape[0], k_pages.shape[1]
        if v_pages.dim() != 4 or tuple(v_pages.shape) != (n_p, h_p, d, BLOCK) or v_pages.stride(3) != 1:
            raise ValueError("dim-major v_pages must be [n_pages][Hkv][d][64] with the token dimension contiguous")
    else:
        raise ValueError("v_layout must be 'token' or 'dim'")
    if k_pages.stride(3) != 1:
        raise ValueError("the head dimension of the pages must be contiguous")
    n_pages, Hkv = k_pages.shape[0], k_pages.shape[1]
    for t, nm in ((page_map, "page_map"), (tables, "tables"), (counts, "counts"), (cu_q, "cu_q"),
                  (prefix_len, "prefix_len")):
        _i32(t, nm)
    B = prefix_len.numel()
    if cu_q.numel() != B + 1 or counts.numel() != B * Hkv or page_map.dim() != 2 or page_map.shape[0] != B:
        raise ValueError("inconsistent B across cu_q / prefix_len / counts / page_map")
    if tables.dim() != 3 or tables.shape[0] != B or tables.shape[1] != Hkv:
        raise ValueError("tables must be [B][Hkv][cap] (B sequences, Hkv KV groups)")
    cap = tables.shape[2]
    dev = _on(_cuda_device(q, "q"), k_pages=k_pages, v_pages=v_pages, page_map=page_map, tables=tables,
              counts=counts, cu_q=cu_q, prefix_len=prefix_len)
    max_chunk_len = _chunk_cap(cu_q, max_chunk_len, stream, dev)
    if auto:
        # the split kernel takes bf16 or fp8 pools whose rows (tokens, or dims of dim-major V)
        # are at most 2^24 elements apart
        splittable = q.dtype == torch.bfloat16 and max(k_pages.stride(2), v_pages.stride(2)) <= (1 << 24)
        n_cus = torch.cuda.get_device_properties(dev).multi_processor_count
        split_pages = plan_split_pages(B, Hq, Hkv, max_chunk_len, cap, n_cus) if splittable else 0
    out, lse = _out_buffers(out, lse, return_lse, q, dev)
    with torch.cuda.device(dev):
        hs = _stream(stream, dev)
        args = (_ptr(q), _DTYPES[q.dtype], _ptr(k_pages), _ptr(v_pages), k_pages.stride(0), k_pages.stride(1),
                k_pages.stride(2), n_pages, _ptr(page_map), page_map.shape[1], _ptr(tables), cap, _ptr(counts),
                _ptr(cu_q), _ptr(prefix_len), B, Hq, Hkv, d, int(max_chunk_len), _scale(sm_scale), _ptr(out),
                _ptr(lse))
        split = bool(split_pages and split_pages > 0)
        if split:
            need = split_workspace_bytes(Tq, Hq, d, cap, split_pages)
            if workspace is None:
                workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            _on(dev, workspace=workspace)
        if fp8:
            st = load().cpa_chunked_prefill_fp8kv(
                _ptr(q), _ptr(k_pages), _ptr(v_pages), k_pages.stride(0), k_pages.stride(1), k_pages.stride(2),
                1 if v_layout == "dim" else 0, v_pages.stride(0), v_pages.stride(1), v_pages.stride(2), float(k_scale),
                float(v_scale), n_pages, _ptr(page_map), page_map.shape[1], _ptr(tables), cap, _ptr(counts), _ptr(cu_q),
                _ptr(prefix_len), B, Hq, Hkv, d, int(max_chunk_len), _scale(sm_scale), _ptr(out), _ptr(lse), Tq,
                int(split_pages) if split else 0, _ptr(workspace) if split else None,
                workspace.numel() * workspace.element_size() if split else 0, hs)
            if st != 0:
                raise CpaError(st, "cpa_chunked_prefill_fp8kv")
            return out, lse
        if v_layout == "dim":
            st = load().cpa_chunked_prefill_vt(
                _ptr(q), _DTYPES[q.dtype], _ptr(k_pages), k_pages.stride(0), k_pages.stride(1), k_pages.stride(2),
                _ptr(v_pages), v_pages.stride(0), v_pages.stride(1), v_pages.stride(2), n_pages, _ptr(page_map),
                page_map.shape[1], _ptr(tables), cap, _ptr(counts), _ptr(cu_q), _ptr(prefix_len), B, Hq, Hkv, d,
                int(max_chunk_len), _scale(sm_scale), _ptr(out), _ptr(lse), Tq, int(split_pages) if split else 0,
                _ptr(workspace) if split else None,
                workspace.numel() * workspace.element_size() if split else 0, hs)
            if st != 0:
                raise CpaError(st, "cpa_chunked_prefill_vt")
            return out, lse
        if split:
            st = load().cpa_chunked_prefill_split(*args, Tq, int(split_pages), _ptr(workspace),
                                                  workspace.numel() * workspace.element_size(), hs)
            if st != 0:
                raise CpaError(st, "cpa_chunked_prefill_split")
            return out, lse
        st = load().cpa_chunked_prefill(*args, hs)
        if st != 0:
            raise CpaError(st, "cpa_chunked_prefill")
        return out, lse


def chunked_prefill_fused(q, k_pages, v_pages, page_map, masks, cu_q, prefix_len, max_chunk_len=None, sm_scale=None,
                          out=None, lse=None, return_lse=False, stream=None, v_layout="token", split_pages=0,
                          workspace=None, nkvb_max=None, k_scale=1.0, v_scale=1.0):
    """The table build and the prefill in one launch (cpa_chunked_prefill_fused): every
    workgroup ORs its KV group's rows of masks (uint8 [B][Hq][nqb_max][nkvb_max]) itself, with
    prefix_blocks = prefix_len / 64 and chunk_blocks = ceil(chunk length / 64).  Bitwise the
    result of build_block_tables followed by chunked_prefill on the same inputs (tables of
    capacity nkvb_max).  bf16 q; bf16 pools, or float8_e4m3fn pools with the dequantization
    scales k_scale / v_scale as chunked_prefill takes them; k_pages / v_pages / v_layout as in
    chunked_prefill.
    Bit-packed masks (int64 [B][Hq][nqb_max][mask_words], as build_block_tables_bits takes them)
    need nkvb_max and run cpa_chunked_prefill_fused_bits.
    split_pages > 0 (or "auto") runs split-KV as chunked_prefill does, with nkvb_max as the table
    capacity; the workspace is allocated here when not given.  max_chunk_len as in chunked_prefill."""
    auto = isinstance(split_pages, str)
    if auto and split_pages != "auto":
        raise ValueError('split_pages must be an int or "auto"')
    if (q.dtype != torch.bfloat16 or k_pages.dtype not in (torch.bfloat16, torch.float8_e4m3fn)
            or v_pages.dtype != k_pages.dtype):
        raise TypeError("the fused path runs a bf16 q over bf16 or float8_e4m3fn k_pages and v_pages")
    if q.dim() != 3 or not q.is_contiguous():
        raise TypeError("q must be a contiguous [Tq][Hq][d] tensor")
    Tq, Hq, d = q.shape
    if k_pages.dim() != 4 or k_pages.shape[2] != BLOCK or k_pages.shape[3] != d or k_pages.stride(3) != 1:
        raise ValueError("k_pages must be [n_pages][Hkv][64][d] with d contiguous")
    n_pages, Hkv = k_pages.shape[0], k_pages.shape[1]
    if v_layout == "token":
        vshape = (n_pages, Hkv, BLOCK, d)
    elif v_layout == "dim":
        vshape = (n_pages, Hkv, d, BLOCK)
    else:
        raise ValueError("v_layout must be 'token' or 'dim'")
    if v_pages.dim() != 4 or tuple(v_pages.shape) != vshape or v_pages.stride(3) != 1:
        raise ValueError(f"v_pages must be {list(vshape)} with the last dimension contiguous")
    if not (isinstance(masks, torch.Tensor) and masks.dtype in (torch.uint8, torch.int64) and masks.dim() == 4
            and masks.is_contiguous()):
        raise TypeError("masks must be a contiguous uint8 [B][Hq][nqb_max][nkvb_max] or int64 "
                        "[B][Hq][nqb_max][mask_words] (bit-packed) tensor")
    bits = masks.dtype == torch.int64
    if bits and nkvb_max is None:
        raise ValueError("bit-packed masks need nkvb_max")
    for t, nm in ((page_map, "page_map"), (cu_q, "cu_q"), (prefix_len, "prefix_len")):
        _i32(t, nm)
    B = prefix_len.numel()
    if masks.shape[0] != B or masks.shape[1] != Hq:
        raise ValueError("masks must be [B][Hq][nqb_max][nkvb_max] (B sequences, Hq query heads)")
    if cu_q.numel() != B + 1 or page_map.dim() != 2 or page_map.shape[0] != B:
        raise ValueError("inconsistent B across cu_q / prefix_len / page_map / masks")
    dev = _on(_cuda_device(q, "q"), k_pages=k_pages, v_pages=v_pages, page_map=page_map, masks=masks, cu_q=cu_q,
              prefix_len=prefix_len)
    max_chunk_len = _chunk_cap(cu_q, max_chunk_len, stream, dev)
    nqb_max = masks.shape[2]
    nkvb_max = int(nkvb_max) if bits else masks.shape[3]
    if auto:
        splittable = max(k_pages.stride(2), v_pages.stride(2)) <= (1 << 24)
        n_cus = torch.cuda.get_device_properties(dev).multi_processor_count
        split_pages = plan_split_pages(B, Hq, Hkv, max_chunk_len, nkvb_max, n_cus) if splittable else 0
    split = bool(split_pages and split_pages > 0)
    out, lse = _out_buffers(out, lse, return_lse, q, dev)
    with torch.cuda.device(dev):
        if split:
            need = split_workspace_bytes(Tq, Hq, d, nkvb_max, split_pages)
            if workspace is None:
                workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            _on(dev, workspace=workspace)
        head = (_ptr(q), BF16, _ptr(k_pages), k_pages.stride(0), k_pages.stride(1), k_pages.stride(2),
                _ptr(v_pages), 1 if v_layout == "dim" else 0, v_pages.stride(0), v_pages.stride(1), v_pages.stride(2),
                _KV_DTYPES[k_pages.dtype], float(k_scale), float(v_scale), n_pages, _ptr(page_map),
                page_map.shape[1], _ptr(masks), nqb_max, nkvb_max)
        tail = (_ptr(cu_q), _ptr(prefix_len), B, Hq, Hkv, d, int(max_chunk_len), _scale(sm_scale), _ptr(out),
                _ptr(lse), Tq, int(split_pages) if split else 0, _ptr(workspace) if split else None,
                workspace.numel() * workspace.element_size() if split else 0, _stream(stream, dev))
        if bits:
            name = "cpa_chunked_prefill_fused_bits"
            st = load().cpa_chunked_prefill_fused_bits(*head, masks.shape[3], *tail)
        else:
            name = "cpa_chunked_prefill_fused"
            st = load().cpa_chunked_prefill_fused(*head, *tail)
    if st != 0:
        raise CpaError(st, name)
    return out, lse


STATIC_SCRATCH_BYTES = 64 * 1024 * 1024   # CPA_STATIC_SCRATCH_BYTES


def chunked_prefill_split_static(q, k_pages, v_pages, page_map, tables, counts, cu_q, prefix_len, max_chunk_len,
                                 split_pages, sm_scale=None, out=None, lse=None, return_lse=False, stream=None):
    """Split-KV attention (token-major V pools, bf16) whose partials live in the library's own
    per-device array instead of a workspace (cpa_chunked_prefill_split_static): the call
    allocates nothing when out (and lse, if wanted) are given.  Same results as
    chunked_prefill(..., split_pages=split_pages)."""
    if q.dtype != torch.bfloat16 or k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("the split path runs bf16 q, k_pages and v_pages")
    if q.dim() != 3 or not q.is_contiguous():
        raise TypeError("q must be a contiguous [Tq][Hq][d] tensor")
    Tq, Hq, d = q.shape
    if k_pages.dim() != 4 or k_pages.shape[2] != BLOCK or k_pages.shape[3] != d or k_pages.stride(3) != 1:
        raise ValueError("k_pages must be [n_pages][Hkv][64][d] with d contiguous")
    if v_pages.shape != k_pages.shape or v_pages.stride() != k_pages.stride():
        raise ValueError("v_pages must match k_pages in shape and strides")
    n_pages, Hkv = k_pages.shape[0], k_pages.shape[1]
    for t, nm in ((page_map, "page_map"), (tables, "tables"), (counts, "counts"), (cu_q, "cu_q"),
                  (prefix_len, "prefix_len")):
        _i32(t, nm)
    B = prefix_len.numel()
    if cu_q.numel() != B + 1 or counts.numel() != B * Hkv or page_map.dim() != 2 or page_map.shape[0] != B:
        raise ValueError("inconsistent B across cu_q / prefix_len / counts / page_map")
    if tables.dim() != 3 or tables.shape[0] != B or tables.shape[1] != Hkv:
        raise ValueError("tables must be [B][Hkv][cap] (B sequences, Hkv KV groups)")
    cap = tables.shape[2]
    dev = _on(_cuda_device(q, "q"), k_pages=k_pages, v_pages=v_pages, page_map=page_map, tables=tables,
              counts=counts, cu_q=cu_q, prefix_len=prefix_len)
    out, lse = _out_buffers(out, lse, return_lse, q, dev)
    with torch.cuda.device(dev):
        st = load().cpa_chunked_prefill_split_static(
            _ptr(q), BF16, _ptr(k_pages), _ptr(v_pages), k_pages.stride(0), k_pages.stride(1), k_pages.stride(2),
            n_pages, _ptr(page_map), page_map.shape[1], _ptr(tables), cap, _ptr(counts), _ptr(cu_q),
            _ptr(prefix_len), B, Hq, Hkv, d, int(max_chunk_len), _scale(sm_scale), _ptr(out), _ptr(lse), Tq,
            int(split_pages), _stream(stream, dev))
    if st != 0:
        raise CpaError(st, "cpa_chunked_prefill_split_static")
    return out, lse


def append_kv(k_new, v_new, k_pages, v_pages, page_map, cu_q, prefix_len, max_chunk_len=None, v_layout="token",
              stream=None):
    """Write each sequence's chunk rows k_new / v_new [Tq][Hkv][d] into their slots of the paged
    pools in place (cpa_append_kv).  k_pages [n_pages][Hkv][64][d]; v_pages the same (v_layout
    "token") or [n_pages][Hkv][d][64] (v_layout "dim"), strided views allowed as in
    chunked_prefill; max_chunk_len as there."""
    if k_new.dtype not in _KV_DTYPES or v_new.dtype != k_new.dtype or k_pages.dtype != k_new.dtype \
            or v_pages.dtype != k_new.dtype:
        raise TypeError("k_new, v_new and the pools must share dtype float32, bfloat16 or float8_e4m3fn")
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        if not (t.is_cuda and t.dim() == 3 and t.is_contiguous()):
            raise TypeError(f"{n} must be a contiguous [Tq][Hkv][d] CUDA tensor")
    if v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must have the same shape")
    dev = _on(k_new.device, v_new=v_new, k_pages=k_pages, v_pages=v_pages)
    Tq, Hkv, d = k_new.shape
    if k_pages.dim() != 4 or tuple(k_pages.shape[1:]) != (Hkv, BLOCK, d) or k_pages.stride(3) != 1:
        raise ValueError("k_pages must be [n_pages][Hkv][64][d] with d contiguous")
    if v_layout == "token":
        vshape = (k_pages.shape[0], Hkv, BLOCK, d)
    elif v_layout == "dim":
        vshape = (k_pages.shape[0], Hkv, d, BLOCK)
    else:
        raise ValueError("v_layout must be 'token' or 'dim'")
    if tuple(v_pages.shape) != vshape or v_pages.stride(3) != 1:
        raise ValueError(f"v_pages must be {list(vshape)} with the last dimension contiguous")
    _dev_i32(page_map, "page_map")
    _dev_i32(cu_q, "cu_q")
    _dev_i32(prefix_len, "prefix_len")
    B = prefix_len.numel()
    if cu_q.numel() != B + 1 or page_map.dim() != 2 or page_map.shape[0] != B:
        raise ValueError("inconsistent B across cu_q / prefix_len / page_map")
    _on(dev, page_map=page_map, cu_q=cu_q, prefix_len=prefix_len)
    max_chunk_len = _chunk_cap(cu_q, max_chunk_len, stream, dev)
    with torch.cuda.device(dev):
        st = load().cpa_append_kv(_ptr(k_new), _ptr(v_new), _KV_DTYPES[k_new.dtype], _ptr(k_pages),
                                  k_pages.stride(0), k_pages.stride(1), k_pages.stride(2), _ptr(v_pages),
                                  1 if v_layout == "dim" else 0, v_pages.stride(0), v_pages.stride(1),
                                  v_pages.stride(2), k_pages.shape[0], _ptr(page_map), page_map.shape[1], _ptr(cu_q),
                                  _ptr(prefix_len), B, Hkv, d, int(max_chunk_len), _stream(stream, dev))
    if st != 0:
        raise CpaError(st, "cpa_append_kv")


def status_string(code: int) -> str:
    return load().cpa_status_string(int(code)).decode()


def version() -> int:
    return load().cpa_version()


def attention_flops(tables, counts, prefix_len, chunk_len, Hq, Hkv, d):
    """Selected-block attention FLOPs, 4*d per causally visible (query, key) pair summed over
    every query head, from host copies (numpy) of the tables.  Only pairs with key position
    <= query position count (a diagonal block contributes 64*65/2 pairs per query block)."""
    import numpy as np
    G = Hq // Hkv
    total = 0
    for b in range(len(prefix_len)):
        P, C = int(prefix_len[b]), int(chunk_len[b])
        r = np.arange(C, dtype=np.int64)
        for g in range(Hkv):
            ids = np.asarray(tables[b, g, :counts[b, g]], dtype=np.int64)
            full = ids[ids * BLOCK + BLOCK - 1 <= P]          # blocks wholly before the chunk
            pairs = int(full.size) * BLOCK * C
            for kb in ids[ids * BLOCK + BLOCK - 1 > P]:
                pairs += int(np.clip(P + r - kb * BLOCK + 1, 0, BLOCK).sum())
            total += pairs * G
    return 4 * d * total
