"""Benchmark of the Block-Union KV Selection hot path on one MI355X.

One step = the whole path over one batch: the table build (masks -> per-group KV block tables)
and the chunked-prefill attention over those tables, both through the C ABI.  Default workload:
the last 2048-token chunk of a 131072-token sequence (prefix 129024), LLaMA-3.1-8B
attention-layer shape (32 query heads, 8 KV heads, head dim 128), bf16, structured per-head
block masks (vertical stripes, slash diagonals, Bernoulli noise, sink block and a 4-block local
window), K/V in a randomly permuted paged pool.  Other workloads: --workload c2 (32K context),
c4 (the full chunked prefill of one 131072-token sequence: 64 chunks of 2048, one step = all 64
chunks in order), c4b (the same 64 chunks as one varlen launch pair), c5a / c5b (varlen batch of four sequences, last 4096-token chunks), c3s (one KV
group's share of the 128K workload, too few tiles for the GPU: run with split-KV, the unsplit
time reported beside it).  All inputs are seeded synthetic data resident in HBM before the timed
region.

Prints one JSON line: selected-block attention TFLOP/s of the whole step, the speedup over the
same kernels run with all-ones masks (dense), the roofline of the dominant kernel (prefill,
timed with HIP events on the stream it runs on) and the CPU oracle timed on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published

WORKLOADS = {
    "c3": ("c3_128k_last_chunk", "128K context, last chunk 2048: prefix 129024 + chunk 2048, "
           "Hq 32 / Hkv 8 / d 128, bf16, structured masks"),
    "c2": ("c2_32k_bf16", "32K context: prefix 30720 + chunk 2048, Hq 32 / Hkv 8 / d 128, bf16, "
           "Bernoulli(0.1) masks + sink + 4-block local"),
    "c4": ("c4_128k_chunked", "full chunked prefill of one 131072-token sequence: 64 chunks of "
           "2048, Hq 32 / Hkv 8 / d 128, bf16, structured masks per chunk"),
    "c5a": ("c5a_varlen_shared", "varlen 4 x last 4096 of {8K,32K,64K,128K}, Hq 32 / Hkv 8 / "
            "d 128, bf16, group-shared stripes 0.1"),
    "c5b": ("c5b_varlen_independent", "varlen 4 x last 4096 of {8K,32K,64K,128K}, Hq 32 / Hkv 8 / "
            "d 128, bf16, per-head stripes 0.1"),
    "c4b": ("c4_128k_chunked_batch", "full chunked prefill of one 131072-token sequence as one varlen "
            "launch pair over its 64 chunks of 2048 (prefix 2048k), Hq 32 / Hkv 8 / d 128, bf16, "
            "structured masks per chunk"),
    "c3s": ("c3s_128k_one_group", "one KV group's share of the 128K last chunk (the per-GPU share of "
            "an 8-way head split): prefix 129024 + chunk 2048, Hq 4 / Hkv 1 / d 128, bf16, "
            "structured masks, split-KV"),
    "c3d": ("c3d_128k_no_noise", "diagnostic: the 128K last chunk (prefix 129024 + chunk 2048, Hq 32 / "
            "Hkv 8 / d 128, bf16) with the headline's stripes, slashes, sink and local window but "
            "without its Bernoulli(0.02) noise term, so the group unions stay sparse"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def hardware_info(dev):
    """The device the line was measured on (with the peak engine clock HIP reports), and the host
    CPU the oracle ran on."""
    import torch
    from sparse_attention_long_reduce_amd import diag
    p = torch.cuda.get_device_properties(dev)
    info = {"gpu": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1)}
    eng_khz, wall_khz = diag.clock_rates(dev.index or 0)
    info["max_engine_clock_mhz"] = round(eng_khz / 1000)
    info["wall_clock_mhz"] = round(wall_khz / 1000, 3)
    try:
        with open("/proc/cpuinfo") as f:
            info["host_cpu"] = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return info


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("prefill_bf16.hip", "prefill_common.h", "cpa_internal.h"):
        with open(os.path.join(ROOT, "sparse_attention_long_reduce_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload_key, v_layout):
    """HBM bytes per prefill launch from the committed rocprofv3 counter summary, or None when
    the summary is absent, covers the other V layout or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"prefill_{workload_key}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_source_hash() or t.get("v_layout", "token") != v_layout:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, max_seconds=15.0):
    """The fp64 oracle (tables in full + attention on a bounded row sample) on all host cores:
    the BLAS pool is set to os.cpu_count() threads for the run (numpy's other operations run on
    one thread); the attention leg uses the oracle's own tables."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle
    host_cores = os.cpu_count() or 1
    default_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    with threadpool_limits(limits=host_cores, user_api="blas"):
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        r = _cpu_baseline_run(w, max_seconds, np, oracle)
    r["cores"] = int(threads)
    r["host_cores"] = int(host_cores)
    r["blas_threads_default"] = int(default_threads)
    return r


def _cpu_baseline_run(w, max_seconds, np, oracle):
    t0 = time.perf_counter()
    T, C = oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    t_tab = time.perf_counter() - t0
    # whole query blocks of one KV group's heads, longest sequence and last blocks first
    flops = 0
    t_att = 0.0
    n_rows = 0
    b = int(np.argmax(w.prefix_len + w.chunk_len))
    C_b = int(w.chunk_len[b])
    done = False
    for g in range(w.Hkv):
        for qi in range((C_b + 63) // 64 - 1, -1, -1):
            rows = np.arange(64 * qi, min(C_b, 64 * qi + 64))
            S = np.array([(b, h, r) for h in range(g * w.G, (g + 1) * w.G) for r in rows], dtype=np.int64)
            t0 = time.perf_counter()
            _, _, nv = oracle.attention_rows(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q,
                                             w.prefix_len, w.Hkv, S, return_nvis=True)
            t_att += time.perf_counter() - t0
            flops += 4 * w.d * int(nv.sum())
            n_rows += len(S)
            if t_att + t_tab > max_seconds:
                done = True
                break
        if done:
            break
    secs = t_tab + t_att
    return {"value": round(flops / secs / 1e12, 5), "unit": "TFLOP/s", "kind": "oracle",
            "sample": f"numpy fp64 oracle: table build for the whole batch ({t_tab:.2f} s) + attention over its "
                      f"own tables for {n_rows} query rows (whole query blocks of KV groups in order, last blocks "
                      f"first) of sequence {b} ({t_att:.2f} s); value = selected FLOPs of those rows / wall time",
            "seconds": round(secs, 3)}


class Batch:
    """One launch pair (table build + prefill) with its inputs resident on the device."""

    def __init__(self, w, dev, kp=None, vp=None, split=False):
        import torch
        import sparse_attention_long_reduce_amd as cpa
        bf = torch.bfloat16
        self.w = w
        self.masks = torch.from_numpy(w.masks).to(dev)
        self.masks_dense = torch.ones_like(self.masks)   # entries outside the causal region are ignored
        self.pb = torch.from_numpy(w.prefix_blocks).to(dev)
        self.cb = torch.from_numpy(w.chunk_blocks).to(dev)
        self.q = torch.from_numpy(w.q).to(dev).to(bf)
        self.kp = torch.from_numpy(w.k_pages).to(dev).to(bf) if kp is None else kp
        self.vp = torch.from_numpy(w.v_pages).to(dev).to(bf) if vp is None else vp
        self.pm = torch.from_numpy(w.page_map).to(dev)
        self.cu = torch.from_numpy(w.cu_q).to(dev)
        self.pl = torch.from_numpy(w.prefix_len).to(dev)
        self.tables = torch.empty((w.B, w.Hkv, w.nkvb_max), dtype=torch.int32, device=dev)
        self.counts = torch.empty((w.B, w.Hkv), dtype=torch.int32, device=dev)
        self.tables_dense = torch.empty_like(self.tables)
        self.counts_dense = torch.empty_like(self.counts)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((self.q.shape[0], w.Hq), dtype=torch.float32, device=dev)
        self.split_pages = 0
        self.workspace = None
        self.v_layout = "token"
        self.vp_dim = None         # dim-major copy of the V pool ([page][group][d][64])
        if split:
            n_cus = torch.cuda.get_device_properties(dev).multi_processor_count
            self.split_pages = cpa.plan_split_pages(w.B, w.Hq, w.Hkv, w.max_chunk_len, w.nkvb_max, n_cus)
            need = cpa.split_workspace_bytes(self.q.shape[0], w.Hq, w.d, w.nkvb_max, self.split_pages)
            self.workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def build(self, cpa, dense):
        if dense:
            cpa.build_block_tables(self.masks_dense, self.pb, self.cb, self.w.Hkv,
                                   tables=self.tables_dense, counts=self.counts_dense)
        else:
            cpa.build_block_tables(self.masks, self.pb, self.cb, self.w.Hkv,
                                   tables=self.tables, counts=self.counts)

    def prefill(self, cpa, dense):
        t, c = (self.tables_dense, self.counts_dense) if dense else (self.tables, self.counts)
        dim = self.v_layout == "dim"
        cpa.chunked_prefill(self.q, self.kp, self.vp_dim if dim else self.vp, self.pm, t, c, self.cu, self.pl,
                            self.w.max_chunk_len, out=self.out, lse=self.lse,
                            split_pages=self.split_pages, workspace=self.workspace, v_layout=self.v_layout)

    def flops(self, cpa, dense=False):
        w = self.w
        t, c = (self.tables_dense, self.counts_dense) if dense else (self.tables, self.counts)
        return cpa.attention_flops(t.cpu().numpy(), c.cpu().numpy(), w.prefix_len,
                                   w.chunk_len, w.Hq, w.Hkv, w.d)


def make_batches(key, dev, v_layouts):
    from workloads import make_config
    from workloads.configs import chunked_sequence_batch, chunked_sequence_chunk
    name, _ = WORKLOADS[key]
    if key == "c4b":
        batches = [Batch(chunked_sequence_batch(), dev)]
    elif key != "c4":
        batches = [Batch(make_config(name), dev, split=(key == "c3s"))]
    else:
        batches = []
        kp = vp = None
        for k in range(64):
            w = chunked_sequence_chunk(k)
            bt = Batch(w, dev, kp, vp)
            kp, vp = bt.kp, bt.vp     # one paged pool shared by all chunks of the sequence
            batches.append(bt)
    if "dim" in v_layouts:
        vp_dim = batches[0].vp.transpose(2, 3).contiguous()   # the same values, dim-major pages
        for bt in batches:
            bt.vp_dim = vp_dim
    for bt in batches:
        bt.v_layout = v_layouts[0]
    return batches


def timed(cpa, batches, modes, steps, warmup):
    """Runs warmup + steps steps; a step runs every launch pair of the workload once for each
    mode in `modes` (False = the workload's masks, True = all-ones masks), the modes taking turns
    so that both see the same clock and thermal state.  HIP events around every launch on torch's
    current stream (the stream the library launches on).  Returns one summary per mode."""
    import numpy as np
    import torch
    for _ in range(warmup):
        for dense in modes:
            for bt in batches:
                bt.build(cpa, dense)
                bt.prefill(cpa, dense)
    torch.cuda.synchronize()
    nb, nm = len(batches), len(modes)
    ev = [[[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nb)] for _ in range(nm)]
          for _ in range(steps)]
    for s in range(steps):
        for m, dense in enumerate(modes):
            for i, bt in enumerate(batches):
                ev[s][m][i][0].record()
                bt.build(cpa, dense)
                ev[s][m][i][1].record()
                bt.prefill(cpa, dense)
                ev[s][m][i][2].record()
    torch.cuda.synchronize()
    out = []
    for m in range(nm):
        build = np.array([[e[0].elapsed_time(e[1]) for e in ev[s][m]] for s in range(steps)])   # ms
        pre = np.array([[e[1].elapsed_time(e[2]) for e in ev[s][m]] for s in range(steps)])
        step = np.array([ev[s][m][0][0].elapsed_time(ev[s][m][-1][2]) for s in range(steps)])
        out.append({"step_ms": float(step.mean()), "step_ms_median": float(np.median(step)),
                    "step_ms_min": float(step.min()), "build_ms": float(build.sum(1).mean()),
                    "build_ms_median": float(np.median(build.sum(1))), "build_ms_min": float(build.sum(1).min()),
                    "prefill_ms": float(pre.sum(1).mean()), "prefill_ms_median": float(np.median(pre.sum(1))),
                    "prefill_ms_min": float(pre.sum(1).min()),
                    "prefill_launch_ms": float(pre.mean()), "launches_per_step": nb})
    return out


def time_direct(cpa, bt, steps, warmup=3):
    """The direct block-sparse baseline on the batch's inputs: per-(head, query block) plans
    (cpa_build_block_plans) and the prefill over them (cpa_chunked_prefill_direct), HIP events
    around each launch; its FLOPs are those of the plans."""
    import numpy as np
    import torch
    w = bt.w
    if bt.vp_dim is None:
        bt.vp_dim = bt.vp.transpose(2, 3).contiguous()
    plans = torch.empty((w.B, w.Hq, w.nqb_max, w.nkvb_max), dtype=torch.int32, device=bt.q.device)
    counts = torch.empty((w.B, w.Hq, w.nqb_max), dtype=torch.int32, device=bt.q.device)
    out = torch.empty_like(bt.q)

    def run():
        cpa.build_block_plans(bt.masks, bt.pb, bt.cb, plans=plans, plan_counts=counts)
        cpa.chunked_prefill_direct(bt.q, bt.kp, bt.vp_dim, bt.pm, plans, counts, bt.cu, bt.pl, w.max_chunk_len,
                                   out=out)

    for _ in range(warmup):
        run()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        cpa.build_block_plans(bt.masks, bt.pb, bt.cb, plans=plans, plan_counts=counts)
        e[1].record()
        cpa.chunked_prefill_direct(bt.q, bt.kp, bt.vp_dim, bt.pm, plans, counts, bt.cu, bt.pl, w.max_chunk_len,
                                   out=out)
        e[2].record()
    torch.cuda.synchronize()
    build = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    pre = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    flop = cpa.plan_flops(plans.cpu().numpy(), counts.cpu().numpy(), w.prefix_len, w.chunk_len, w.d)
    n_blk = int(counts.sum())
    # each plan block's K and V (64 tokens x d, bf16) reach the registers of its tile once
    opb = n_blk * 2 * 64 * w.d * 2
    return {"plan_build_us": round(build * 1e3, 2), "prefill_ms": round(pre, 4), "step_ms": round(build + pre, 4),
            "flop": int(flop), "prefill_tflops": round(flop / (pre * 1e-3) / 1e12, 2), "plan_blocks": n_blk,
            "roofline": {"bound": "hbm", "achieved": round(opb / (pre * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(opb / (pre * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": opb,
                         "note": "K/V operand bytes of the plans, one read per (head, query block) tile"}}


def time_fused(cpa, batches, steps, warmup=3):
    """The table build moved into the prefill's prologue (cpa_chunked_prefill_fused, one launch
    per launch pair) against the separate table-build + prefill launches on the same inputs.
    The two take turns step by step, so that both see the same clock and thermal state; HIP
    events around each step.  Also checks that their outputs are equal bit for bit."""
    import numpy as np
    import torch
    from workloads.configs import pack_mask_bits
    outs = [torch.empty_like(bt.q) for bt in batches]
    lses = [torch.empty_like(bt.lse) for bt in batches]
    outs_b = [torch.empty_like(bt.q) for bt in batches]
    lses_b = [torch.empty_like(bt.lse) for bt in batches]
    bits = [torch.from_numpy(pack_mask_bits(bt.w.masks).view(np.int64)).to(bt.q.device) for bt in batches]

    def fused_step(from_bits=False):
        for i, bt in enumerate(batches):
            dim = bt.v_layout == "dim"
            m, o, l = (bits[i], outs_b[i], lses_b[i]) if from_bits else (bt.masks, outs[i], lses[i])
            cpa.chunked_prefill_fused(bt.q, bt.kp, bt.vp_dim if dim else bt.vp, bt.pm, m, bt.cu, bt.pl,
                                      bt.w.max_chunk_len, out=o, lse=l, v_layout=bt.v_layout,
                                      split_pages=bt.split_pages, workspace=bt.workspace,
                                      nkvb_max=bt.w.nkvb_max if from_bits else None)

    def separate_step():
        for bt in batches:
            bt.build(cpa, False)
            bt.prefill(cpa, False)

    for _ in range(warmup):
        separate_step()
        fused_step()
        fused_step(True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        separate_step()
        e[1].record()
        e[2].record()
        fused_step()
        e[3].record()
        e[4].record()
        fused_step(True)
        e[5].record()
    torch.cuda.synchronize()
    sep = np.array([e[0].elapsed_time(e[1]) for e in ev])
    fu = np.array([e[2].elapsed_time(e[3]) for e in ev])
    fb = np.array([e[4].elapsed_time(e[5]) for e in ev])

    def same(os_, ls_):
        return all(torch.equal(o.view(torch.int16), bt.out.view(torch.int16))
                   and torch.equal(l.view(torch.int32), bt.lse.view(torch.int32))
                   for o, l, bt in zip(os_, ls_, batches))
    return {"step_ms": float(fu.mean()), "step_ms_median": float(np.median(fu)), "step_ms_min": float(fu.min()),
            "separate_step_ms": float(sep.mean()), "separate_step_ms_median": float(np.median(sep)),
            "bits_step_ms": float(fb.mean()), "launches_per_step": len(batches),
            "outputs_equal_separate": bool(same(outs, lses) and same(outs_b, lses_b))}


def time_graph(cpa, batches, steps):
    """The workload's launch pairs (sparse masks) captured into one HIP graph and replayed; HIP
    events around each replay.  Returns the mean replay time."""
    import numpy as np
    import torch

    def step():
        for bt in batches:
            bt.build(cpa, False)
            bt.prefill(cpa, False)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(2):
        g.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))


def alternate_ms(fns, steps, warmup):
    """HIP-event time of each callable in `fns`, the callables taking turns launch by launch so
    that all of them see the same clock and thermal state (the engine clock follows the power
    drawn, and timing one after the other favours whichever runs in the cooler slot); returns
    the mean ms of each over `steps` turns."""
    import numpy as np
    import torch
    for _ in range(warmup):
        for f in fns:
            f()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(steps)]
    for row in ev:
        for f, (e0, e1) in zip(fns, row):
            e0.record()
            f()
            e1.record()
    torch.cuda.synchronize()
    return [float(np.mean([row[i][0].elapsed_time(row[i][1]) for row in ev])) for i in range(len(fns))]


def time_fp8kv(cpa, bt, steps, warmup=3):
    """The batch's prefill over an fp8 (e4m3) copy of its KV cache, per-tensor scale 1/4
    (cpa_chunked_prefill_fp8kv), with dim-major and with token-major V taking turns, HIP events
    around each launch (and the merge, when the batch runs split-KV: the same ranges as its bf16
    prefill)."""
    import torch
    w = bt.w
    f8 = torch.float8_e4m3fn
    kp8 = (torch.from_numpy(w.k_pages) * 4.0).to(f8).to(bt.q.device)
    vp8 = (torch.from_numpy(w.v_pages) * 4.0).to(f8).to(bt.q.device)
    vp8d = vp8.view(torch.uint8).transpose(2, 3).contiguous().view(f8)   # dim-major copy
    out = torch.empty_like(bt.q)

    def launch(vp, layout):
        def run():
            cpa.chunked_prefill(bt.q, kp8, vp, bt.pm, bt.tables, bt.counts, bt.cu, bt.pl, w.max_chunk_len,
                                out=out, k_scale=0.25, v_scale=0.25, v_layout=layout, split_pages=bt.split_pages,
                                workspace=bt.workspace)
        return run

    ms_dim, ms_tok = alternate_ms([launch(vp8d, "dim"), launch(vp8, "token")], steps, warmup)
    return {"prefill_ms": round(ms_dim, 4), "prefill_ms_token_major_v": round(ms_tok, 4),
            "kv_bytes": int(kp8.numel() + vp8.numel()), "kv_bytes_bf16": int(2 * (kp8.numel() + vp8.numel())),
            "split_pages": int(bt.split_pages),
            "note": "codes staged in LDS and converted to bf16 once per workgroup; token-major V transposed "
                    "by ds_read_b64_tr_b8 on the way" + ("; split-KV ranges and merge as the bf16 prefill"
                                                        if bt.split_pages else "")}


def time_build_bits(cpa, batches, steps):
    """HIP-event time of the table build from bit-packed masks (cpa_build_block_tables_bits) for
    every launch pair of the workload, and whether its tables equal the byte-mask build's."""
    import numpy as np
    import torch
    from workloads.configs import pack_mask_bits
    bits = [torch.from_numpy(pack_mask_bits(bt.w.masks).view(np.int64)).to(bt.q.device) for bt in batches]
    outs = [(torch.empty_like(bt.tables), torch.empty_like(bt.counts)) for bt in batches]

    def run():
        for bt, mb, (t, c) in zip(batches, bits, outs):
            cpa.build_block_tables_bits(mb, bt.w.nkvb_max, bt.pb, bt.cb, bt.w.Hkv, tables=t, counts=c)

    for _ in range(3):
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3
    same = all(torch.equal(t, bt.tables) and torch.equal(c, bt.counts) for bt, (t, c) in zip(batches, outs))
    nbytes = sum(int(b.numel()) * 8 for b in bits)
    tbytes = sum(int(bt.tables.numel() * 4 + bt.counts.numel() * 4) for bt in batches)
    gbs = (nbytes + tbytes) / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "mask_bytes": nbytes, "tables_equal_byte_masks": bool(same),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 5), "algorithmic_bytes": nbytes + tbytes}}


def time_append(cpa, bt, steps, reps=20):
    """Time of cpa_append_kv writing the batch's chunk rows (taken from the pool itself, so the
    pool's contents do not change) into the pool in the bench's V layout.  `us` is the GPU time of
    one call: HIP events around replays of a captured graph of `reps` calls back to back, so the
    host's per-call overhead (the binding's checks) is not in it; `us_eager_call` is the event time
    of one eager call, which includes that overhead whenever the host is slower than the kernel."""
    import numpy as np
    import torch
    w = bt.w
    pos = [w.prefix_len[b] + np.arange(w.chunk_len[b]) for b in range(w.B)]
    pages = torch.from_numpy(np.concatenate([w.page_map[b, p // 64] for b, p in enumerate(pos)]).astype(np.int64))
    slots = torch.from_numpy(np.concatenate([p % 64 for p in pos]).astype(np.int64))
    pages, slots = pages.to(bt.q.device), slots.to(bt.q.device)
    k_rows = bt.kp[pages, :, slots].contiguous()
    v_rows = bt.vp[pages, :, slots].contiguous()
    dim = bt.v_layout == "dim"
    vpool = bt.vp_dim if dim else bt.vp

    def run():
        cpa.append_kv(k_rows, v_rows, bt.kp, vpool, bt.pm, bt.cu, bt.pl, w.max_chunk_len, v_layout=bt.v_layout)

    def event_times(fn, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    eager_us = event_times(run, steps)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side), torch.cuda.graph(graph, stream=side):
        for _ in range(reps):
            run()
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    us = event_times(graph.replay, steps) / reps
    del graph
    nbytes = 2 * 2 * k_rows.numel() * k_rows.element_size()   # K and V, read once and written once
    return {"us": round(us, 2), "us_eager_call": round(eager_us, 2), "rows": int(k_rows.shape[0]),
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": nbytes}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first: the engine clock ramps up over the first ~40 ms of work")
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--v-layout", default="dim", choices=("dim", "token"),
                    help="V pool pages dim-major [page][group][d][64] or token-major [page][group][64][d] "
                         "(K pages are token-major)")
    ap.add_argument("--no-layout-ab", action="store_true",
                    help="skip the timing of the other V layout")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device-to-device copy of 1 GiB three times (the reference "
                         "kernel that scales the HBM byte counters)")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="only run the bf16 MFMA-loop probe (cpa_diag_mfma_loop) and print its rate and the "
                         "engine clock it ran at")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: every figure it reports is one GPU's (the path shards "
              "along KV groups or the sequence with no change to the kernels); --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4}))
        return

    import sparse_attention_long_reduce_amd as cpa
    from sparse_attention_long_reduce_amd import diag

    if args.mfma_peak:
        dev = torch.device("cuda:0")
        out = {}
        for threads in (256, 512):
            r = diag.mfma_peak(dev, threads=threads)
            out[f"waves_per_simd_{threads // 256}"] = {k: (round(v, 3) if isinstance(v, float) else v)
                                                        for k, v in r.items()}
        out["published_peak_tflops"] = MFMA_BF16_PEAK_TFLOPS
        out["hardware"] = hardware_info(dev)
        print(json.dumps(out), flush=True)
        return

    name, desc = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    other = "token" if args.v_layout == "dim" else "dim"
    batches = make_batches(args.workload, dev, (args.v_layout,) if args.no_layout_ab else (args.v_layout, other))
    torch.cuda.synchronize()
    log(f"[bench] {name}: {len(batches)} launch pair(s) per step, inputs resident on the GPU "
        f"({time.perf_counter() - t0:.1f} s)")

    modes = (False,) if args.no_dense else (False, True)
    res = timed(cpa, batches, modes, args.steps, args.warmup)
    r = res[0]
    flops = sum(bt.flops(cpa) for bt in batches)
    union = sum(int(bt.counts.sum()) for bt in batches)
    log(f"[bench] sparse: step {r['step_ms']:.3f} ms, prefill {r['prefill_ms']:.3f} ms, "
        f"build {r['build_ms'] * 1e3:.1f} us, union blocks {union}")
    d = None
    if not args.no_dense:
        d = res[1]
        dflops = sum(bt.flops(cpa, dense=True) for bt in batches)
        log(f"[bench] dense: step {d['step_ms']:.3f} ms, prefill {d['prefill_ms']:.3f} ms")

    unsplit = None
    if any(bt.split_pages for bt in batches):
        saved = [bt.split_pages for bt in batches]
        for bt in batches:
            bt.split_pages = 0
        unsplit = timed(cpa, batches, (False,), max(5, args.steps // 2), 2)[0]
        for bt, sp in zip(batches, saved):
            bt.split_pages = sp
        log(f"[bench] unsplit: prefill {unsplit['prefill_ms']:.3f} ms (split pages {saved[0]})")

    layout_ab = None
    if not args.no_layout_ab:
        # the two V layouts take turns launch by launch (prefill only, the tables built above)
        def in_layout(layout):
            def run():
                for bt in batches:
                    bt.v_layout = layout
                    bt.prefill(cpa, False)
            return run
        ms_main, ms_other = alternate_ms([in_layout(args.v_layout), in_layout(other)], max(5, args.steps // 2), 2)
        for bt in batches:
            bt.v_layout = args.v_layout
        layout_ab = {args.v_layout: round(ms_main, 4), other: round(ms_other, 4)}
        log(f"[bench] V layout A/B prefill ms: {layout_ab}")

    direct = None
    if len(batches) == 1 and batches[0].split_pages == 0:
        direct = time_direct(cpa, batches[0], max(5, args.steps // 2))
        log(f"[bench] direct block-sparse baseline: plans {direct['plan_build_us']:.1f} us, prefill "
            f"{direct['prefill_ms']:.3f} ms ({direct['prefill_tflops']:.0f} TFLOP/s on {direct['flop']:.3e} "
            f"FLOP, {direct['plan_blocks']} plan blocks)")
    fp8kv = None
    if len(batches) == 1:
        fp8kv = time_fp8kv(cpa, batches[0], max(5, args.steps // 2))
        fp8kv["prefill_tflops"] = round(flops / (fp8kv["prefill_ms"] * 1e-3) / 1e12, 2)
        fp8kv["roofline"] = {"bound": "mfma", "achieved": fp8kv["prefill_tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(fp8kv["prefill_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)}
        log(f"[bench] fp8 KV cache: prefill {fp8kv['prefill_ms']:.3f} ms ({fp8kv['prefill_tflops']:.0f} TFLOP/s), "
            f"cache {fp8kv['kv_bytes'] / 2**20:.0f} MiB vs {fp8kv['kv_bytes_bf16'] / 2**20:.0f} MiB bf16")
    fu = time_fused(cpa, batches, max(5, args.steps))   # every workload, split-KV included
    fused = {"step_ms": round(fu["step_ms"], 4), "step_ms_median": round(fu["step_ms_median"], 4),
             "step_ms_min": round(fu["step_ms_min"], 4), "separate_step_ms": round(fu["separate_step_ms"], 4),
             "speedup_over_separate": round(fu["separate_step_ms"] / fu["step_ms"], 4),
             "bit_masks_step_ms": round(fu["bits_step_ms"], 4),
             "launches_per_step": fu["launches_per_step"],
             "outputs_equal_separate": fu["outputs_equal_separate"],
             "note": "cpa_chunked_prefill_fused: each prefill workgroup builds its group's union from the "
                     "masks in its prologue; one launch per launch pair instead of two; timed step by step "
                     "in turn with the separate launches and with the same launch from bit-packed masks "
                     "(cpa_chunked_prefill_fused_bits); outputs_equal_separate covers both"}
    log(f"[bench] fused union in the prefill prologue: step {fu['step_ms']:.3f} ms ({fu['bits_step_ms']:.3f} ms from "
        f"bit masks) vs separate {fu['separate_step_ms']:.3f} ms (in turn), outputs equal: "
        f"{fu['outputs_equal_separate']}")
    bits = time_build_bits(cpa, batches, max(5, args.steps))
    log(f"[bench] table build from bit-packed masks: {bits['us']:.1f} us ({bits['mask_bytes']} mask bytes), "
        f"tables equal: {bits['tables_equal_byte_masks']}")
    graph = None
    if args.workload == "c4":
        gms = time_graph(cpa, batches, max(5, args.steps // 2))
        graph = {"step_ms": round(gms, 4), "eager_step_ms": round(r["step_ms"], 4),
                 "speedup_over_eager": round(r["step_ms"] / gms, 4),
                 "note": "the 64 launch pairs of a step captured into one HIP graph and replayed"}
        log(f"[bench] one HIP graph of the step's {2 * len(batches)} launches: {gms:.3f} ms per replay")
    append = None
    if args.workload != "c4":
        append = time_append(cpa, batches[0], max(5, args.steps))
        log(f"[bench] kv append: {append['us']:.1f} us for {append['rows']} rows, "
            f"{append['roofline']['achieved']:.0f} GB/s")

    w0 = batches[-1].w
    bt0 = batches[0]
    step_tflops = flops / (r["step_ms"] * 1e-3) / 1e12
    pre_tflops = flops / (r["prefill_ms"] * 1e-3) / 1e12
    mask_bytes = sum(int(bt.w.masks.nbytes) for bt in batches)
    tab_bytes = sum(int(bt.tables.numel() * 4 + bt.counts.numel() * 4) for bt in batches)
    context = int(max(int(bt.w.prefix_len.max() + bt.w.chunk_len.max()) for bt in batches))
    result = {
        "metric": "selected-block attention TFLOP/s + speedup vs dense at 128K context, chunk 2048",
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, synthetic block masks, permuted paged KV pool)",
        "config": {"workload": desc, "sequences": int(w0.B), "chunk_len": int(w0.max_chunk_len),
                   "context": context, "Hq": w0.Hq, "Hkv": w0.Hkv, "head_dim": w0.d, "block": 64,
                   "launch_pairs_per_step": len(batches),
                   "kv_layout": "K pages token-major [page][group][64][d], V pages "
                                + ("dim-major [page][group][d][64]" if args.v_layout == "dim"
                                   else "token-major [page][group][64][d]")},
        "selected_flop": int(flops),
        "union_blocks": union,
        "prefill_tflops": round(pre_tflops, 2),
        "prefill_ms": round(r["prefill_ms"], 4),
        "table_build_us": round(r["build_ms"] * 1e3, 2),
        "timing_stats_ms": {"step": {"mean": round(r["step_ms"], 4), "median": round(r["step_ms_median"], 4),
                                     "min": round(r["step_ms_min"], 4)},
                            "prefill": {"mean": round(r["prefill_ms"], 4), "median": round(r["prefill_ms_median"], 4),
                                        "min": round(r["prefill_ms_min"], 4)},
                            "table_build": {"mean": round(r["build_ms"], 5), "median": round(r["build_ms_median"], 5),
                                            "min": round(r["build_ms_min"], 5)},
                            "note": f"over {args.steps} timed steps; value and roofline use the mean"},
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": read_traffic(args.workload, args.v_layout),
                     "kernel": f"prefill_bf16_kernel<128, {'true' if bt0.split_pages else 'false'}, "
                               f"{'true' if args.v_layout == 'dim' else 'false'}, false, false>"},
        "table_build_roofline": {
            "bound": "hbm", "achieved": round((mask_bytes + tab_bytes) / (r["build_ms"] * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round((mask_bytes + tab_bytes) / (r["build_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
            "algorithmic_bytes": mask_bytes + tab_bytes},
    }
    if d is not None:
        result["dense"] = {"step_ms": round(d["step_ms"], 4), "prefill_ms": round(d["prefill_ms"], 4),
                           "flop": int(dflops), "prefill_tflops": round(dflops / (d["prefill_ms"] * 1e-3) / 1e12, 2)}
        result["speedup_vs_dense"] = {"kernel": round(d["prefill_ms"] / r["prefill_ms"], 4),
                                      "end_to_end": round(d["step_ms"] / r["step_ms"], 4)}
    if layout_ab is not None:
        result["v_layout_prefill_ms"] = layout_ab
    if append is not None:
        result["kv_append"] = append
    result["table_build_bit_masks"] = bits
    result["fused_union"] = fused
    if graph is not None:
        result["graph_replay"] = graph
    if fp8kv is not None:
        result["fp8_kv"] = fp8kv
    if direct is not None:
        direct["union_speedup_over_direct"] = round(direct["step_ms"] / r["step_ms"], 4)
        result["direct_block_sparse_baseline"] = direct
    if unsplit is not None:
        result["split_kv"] = {"split_pages": batches[0].split_pages,
                              "unsplit_prefill_ms": round(unsplit["prefill_ms"], 4),
                              "speedup_over_unsplit": round(unsplit["prefill_ms"] / r["prefill_ms"], 4)}
    result["hardware"] = hardware_info(torch.device("cuda", 0))
    # the measured MFMA ceiling of this device: a loop of independent bf16 MFMAs, two waves per SIMD
    mp = diag.mfma_peak(torch.device("cuda", 0))
    result["roofline"]["measured_peak"] = {
        "achieved_tflops": round(mp["tflops"], 1), "engine_clock_mhz": round(mp["engine_clock_mhz"]),
        "frac_of_published": round(mp["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
        "prefill_frac_of_measured": round(pre_tflops / mp["tflops"], 4),
        "note": "cpa_diag_mfma_loop: 4 independent v_mfma_f32_32x32x16_bf16 chains per wave, two waves per SIMD, "
                "one workgroup per CU, no memory traffic; clock = shader cycles / wall-clock ticks of workgroup 0"}
    result["hardware"]["engine_clock_mhz_mfma_loop"] = round(mp["engine_clock_mhz"])
    result["pages_context"] = ("CompactAttention reports up to 2.72x attention speedup at 128K on "
                               "LLaMA-3.1-8B-Instruct (hardware not stated); context only")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        bt = batches[-1]
        result["cpu_baseline"] = cpu_baseline(bt.w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
