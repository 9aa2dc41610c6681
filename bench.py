"""Benchmark of the Block-Union KV Selection hot path on one MI355X.

One step = the whole path over one batch: the table build (masks -> per-group tables) and the
chunked-prefill attention over those tables, both through the C ABI.  Default workload: the last
2048-token chunk of a 131072-token sequence (prefix 129024), LLaMA-3.1-8B attention-layer shape
(32 query heads, 8 KV heads, head dim 128), bf16, structured per-head block masks (vertical
stripes, slash diagonals, Bernoulli noise, sink block and a 4-block local window), K/V in a
randomly permuted paged pool.  All inputs are seeded synthetic data resident in HBM before the
timed region.

Prints one JSON line with the selected-block attention TFLOP/s (whole step), the speedup over
the same kernels run with all-ones masks (dense), the roofline of the dominant kernel (prefill,
measured with HIP events on the stream it runs on) and the CPU oracle timed on a bounded sample.
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
MFMA_F32_PEAK_TFLOPS = 157.3     # MI355X fp32 (no fp32 MFMA headline beyond the vector rate)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published

WORKLOADS = {
    "c3": ("c3_128k_last_chunk", "128K context, last chunk 2048: prefix 129024 + chunk 2048, "
           "Hq 32 / Hkv 8 / d 128, bf16, structured masks"),
    "c2": ("c2_32k_bf16", "32K context: prefix 30720 + chunk 2048, Hq 32 / Hkv 8 / d 128, bf16, "
           "Bernoulli(0.1) masks + sink + 4-block local"),
    "c5a": ("c5a_varlen_shared", "varlen 4 x last 4096 of {8K,32K,64K,128K}, Hq 32 / Hkv 8 / d 128, "
            "bf16, group-shared stripes 0.1"),
    "c5b": ("c5b_varlen_independent", "varlen 4 x last 4096 of {8K,32K,64K,128K}, Hq 32 / Hkv 8 / "
            "d 128, bf16, per-head stripes 0.1"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("prefill_bf16.hip", "prefill_common.h", "cpa_internal.h"):
        with open(os.path.join(ROOT, "sparse_attention_long_reduce_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload_key):
    """HBM bytes per prefill launch from the committed rocprofv3 counter summary, or None when
    the summary is absent or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"prefill_{workload_key}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, T, C, max_seconds=20.0):
    """The fp64 oracle (tables in full + attention on a bounded row sample) on the host cores."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    t0 = time.perf_counter()
    oracle.block_union_tables(w.masks, w.prefix_blocks, w.chunk_blocks, w.Hkv, w.nkvb_max)
    t_tab = time.perf_counter() - t0
    # rows: whole query blocks of group 0's heads, last blocks first (the heaviest), until time runs out
    flops = 0
    t_att = 0.0
    n_rows = 0
    rng = np.random.default_rng(0)
    b = w.B - 1
    C_b = int(w.chunk_len[b])
    for qi in range((C_b + 63) // 64 - 1, -1, -1):
        rows = np.arange(64 * qi, min(C_b, 64 * qi + 64))
        S = np.array([(b, h, r) for h in range(w.G) for r in rows], dtype=np.int64)
        t0 = time.perf_counter()
        _, _, nv = oracle.attention_rows(w.q, w.k_pages, w.v_pages, w.page_map, T, C, w.cu_q,
                                         w.prefix_len, w.Hkv, S, return_nvis=True)
        t_att += time.perf_counter() - t0
        flops += 4 * w.d * int(nv.sum())
        n_rows += len(S)
        if t_att + t_tab > max_seconds:
            break
    del rng
    secs = t_tab + t_att
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"numpy fp64 oracle: full table build ({t_tab:.2f} s) + attention for {n_rows} "
                      f"query rows (group 0's heads, last query blocks first) of sequence {b} "
                      f"({t_att:.2f} s); value = selected FLOPs of those rows / wall time",
            "seconds": round(secs, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device-to-device copy of 1 GiB three times (the reference "
                         "kernel that scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the path is measured on one GPU's share "
              "(see the sharding notes in DESIGN.md); --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
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
    from workloads import make_config

    name, desc = WORKLOADS[args.workload]
    t0 = time.perf_counter()
    w = make_config(name)
    log(f"[bench] generated {name} in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = torch.bfloat16
    masks = torch.from_numpy(w.masks).to(dev)
    masks_dense = torch.ones_like(masks)   # entries outside the causal region are ignored
    pb = torch.from_numpy(w.prefix_blocks).to(dev)
    cb = torch.from_numpy(w.chunk_blocks).to(dev)
    q = torch.from_numpy(w.q).to(dev).to(bf)
    kp = torch.from_numpy(w.k_pages).to(dev).to(bf)
    vp = torch.from_numpy(w.v_pages).to(dev).to(bf)
    pm = torch.from_numpy(w.page_map).to(dev)
    cu = torch.from_numpy(w.cu_q).to(dev)
    pl = torch.from_numpy(w.prefix_len).to(dev)
    tables = torch.empty((w.B, w.Hkv, w.nkvb_max), dtype=torch.int32, device=dev)
    counts = torch.empty((w.B, w.Hkv), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], w.Hq), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("[bench] inputs resident on the GPU")

    def step(m):
        cpa.build_block_tables(m, pb, cb, w.Hkv, tables=tables, counts=counts)
        cpa.chunked_prefill(q, kp, vp, pm, tables, counts, cu, pl, w.max_chunk_len, out=out, lse=lse)

    def timed(m, steps, warmup):
        for _ in range(warmup):
            step(m)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record()
            cpa.build_block_tables(m, pb, cb, w.Hkv, tables=tables, counts=counts)
            ev[i][1].record()
            cpa.chunked_prefill(q, kp, vp, pm, tables, counts, cu, pl, w.max_chunk_len, out=out, lse=lse)
            ev[i][2].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        build_ms = [e[0].elapsed_time(e[1]) for e in ev]
        pre_ms = [e[1].elapsed_time(e[2]) for e in ev]
        total_ms = ev[0][0].elapsed_time(ev[-1][2])
        return {"step_ms": total_ms / steps, "build_ms": float(np.mean(build_ms)),
                "prefill_ms": float(np.mean(pre_ms)), "prefill_ms_median": float(np.median(pre_ms)),
                "prefill_ms_min": float(np.min(pre_ms)), "wall_s": wall}

    # sparse (the method)
    r = timed(masks, args.steps, args.warmup)
    T = tables.cpu().numpy()
    Cn = counts.cpu().numpy()
    flops = cpa.attention_flops(T, Cn, w.prefix_len, w.chunk_len, w.Hq, w.Hkv, w.d)
    log(f"[bench] sparse: step {r['step_ms']:.3f} ms, prefill {r['prefill_ms']:.3f} ms, "
        f"build {r['build_ms'] * 1e3:.1f} us, union blocks {int(Cn.sum())} of "
        f"{int(w.B * w.Hkv * w.nkvb_max)}")
    # dense (all-ones masks through the same kernels)
    d = None
    if not args.no_dense:
        d = timed(masks_dense, max(5, args.steps // 2), 2)
        Td = tables.cpu().numpy()
        Cd = counts.cpu().numpy()
        dflops = cpa.attention_flops(Td, Cd, w.prefix_len, w.chunk_len, w.Hq, w.Hkv, w.d)
        log(f"[bench] dense: step {d['step_ms']:.3f} ms, prefill {d['prefill_ms']:.3f} ms")
        cpa.build_block_tables(masks, pb, cb, w.Hkv, tables=tables, counts=counts)
        torch.cuda.synchronize()

    step_tflops = flops / (r["step_ms"] * 1e-3) / 1e12
    pre_tflops = flops / (r["prefill_ms"] * 1e-3) / 1e12
    mask_bytes = int(w.masks.nbytes)
    tab_bytes = int(T.nbytes + Cn.nbytes)
    traffic = read_traffic(args.workload)
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
        "config": {"workload": desc, "sequences": int(w.B), "chunk_len": int(w.max_chunk_len),
                   "context": int(w.prefix_len.max() + w.max_chunk_len), "Hq": w.Hq, "Hkv": w.Hkv,
                   "head_dim": w.d, "block": 64},
        "selected_flop": int(flops),
        "union_blocks": int(Cn.sum()),
        "prefill_tflops": round(pre_tflops, 2),
        "prefill_ms": round(r["prefill_ms"], 4),
        "table_build_us": round(r["build_ms"] * 1e3, 2),
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel": "prefill_kernel<bf16,128>"},
        "table_build_roofline": {"bound": "hbm", "achieved": round((mask_bytes + tab_bytes) / (r["build_ms"] * 1e-3) / 1e9, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round((mask_bytes + tab_bytes) / (r["build_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
                                 "algorithmic_bytes": mask_bytes + tab_bytes},
    }
    if d is not None:
        result["dense"] = {"step_ms": round(d["step_ms"], 4), "prefill_ms": round(d["prefill_ms"], 4),
                           "flop": int(dflops), "prefill_tflops": round(dflops / (d["prefill_ms"] * 1e-3) / 1e12, 2)}
        result["speedup_vs_dense"] = {"kernel": round(d["prefill_ms"] / r["prefill_ms"], 4),
                                      "end_to_end": round(d["step_ms"] / r["step_ms"], 4)}
    result["pages_context"] = ("CompactAttention reports up to 2.72x attention speedup at 128K on "
                               "LLaMA-3.1-8B-Instruct (hardware not stated); context only")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w, T, Cn)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
