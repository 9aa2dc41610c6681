"""The Python binding refuses, before any call into the library, what would make a kernel read
or write outside its buffers: tensors not on the GPU, and caller-given outputs of the wrong
shape, dtype or layout."""
import pytest
import torch

import sparse_attention_long_reduce_amd as cpa


def _cpu_args(d=64, dtype=torch.bfloat16):
    q = torch.zeros(64, 4, d, dtype=dtype)
    kp = torch.zeros(2, 1, 64, d, dtype=dtype)
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)  # noqa: E731
    return q, kp, kp.clone(), i32(1, 2), i32(1, 1, 2), i32(1, 1), i32(2), i32(1)


def test_prefill_refuses_cpu_tensors():
    q, kp, vp, pm, t, c, cu, pl = _cpu_args()
    with pytest.raises(TypeError, match="CUDA"):
        cpa.chunked_prefill(q, kp, vp, pm, t, c, cu, pl, 64)
    with pytest.raises(TypeError, match="CUDA"):
        cpa.chunked_prefill(q, kp.to(torch.float8_e4m3fn),
                            vp.to(torch.float8_e4m3fn), pm, t, c, cu, pl, 64)


def test_direct_and_append_refuse_cpu_tensors():
    q, kp, vp, pm, t, c, cu, pl = _cpu_args()
    with pytest.raises(TypeError, match="CUDA"):
        cpa.chunked_prefill_direct(q, kp, vp.transpose(2, 3).contiguous(), pm, torch.zeros(1, 4, 1, 2, dtype=torch.int32),
                                   torch.zeros(1, 4, 1, dtype=torch.int32), cu, pl, 64)
    with pytest.raises(TypeError, match="CUDA"):
        cpa.append_kv(torch.zeros(64, 1, 64, dtype=torch.bfloat16), torch.zeros(64, 1, 64, dtype=torch.bfloat16),
                      kp, vp, pm, cu, pl, 64)


def test_table_builds_refuse_cpu_tensors():
    m = torch.zeros(1, 4, 1, 2, dtype=torch.uint8)
    pb = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(TypeError, match="CUDA"):
        cpa.build_block_tables(m, pb, pb, 1)
    with pytest.raises(TypeError, match="CUDA"):
        cpa.build_block_tables_bits(torch.zeros(1, 4, 1, 1, dtype=torch.int64), 2, pb, pb, 1)
    with pytest.raises(TypeError, match="CUDA"):
        cpa.build_block_plans(m, pb, pb)


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_caller_outputs_are_checked():
    q, kp, vp, pm, t, c, cu, pl = [x.cuda() for x in _cpu_args()]
    cu[1] = 64
    with pytest.raises(ValueError, match="out"):
        cpa.chunked_prefill(q, kp, vp, pm, t, c, cu, pl, 64, out=torch.empty(32, 4, 64, dtype=q.dtype, device="cuda"))
    with pytest.raises(ValueError, match="out"):
        cpa.chunked_prefill(q, kp, vp, pm, t, c, cu, pl, 64, out=torch.empty(64, 4, 64, device="cuda"))
    with pytest.raises(ValueError, match="lse"):
        cpa.chunked_prefill(q, kp, vp, pm, t, c, cu, pl, 64, lse=torch.empty(4, 64, device="cuda"))
    with pytest.raises(ValueError, match="lse"):
        cpa.chunked_prefill(q, kp, vp, pm, t, c, cu, pl, 64,
                            lse=torch.empty(64, 4, dtype=torch.float64, device="cuda"))
    with pytest.raises(TypeError, match="CUDA"):
        cpa.chunked_prefill(q, kp, vp, pm, t, c, cu, pl, 64, out=torch.empty(64, 4, 64, dtype=q.dtype))
    # well-formed caller outputs are used as given
    o = torch.empty_like(q)
    lse = torch.empty(64, 4, device="cuda")
    o2, lse2 = cpa.chunked_prefill(q, kp, vp, pm, t, c, cu, pl, 64, out=o, lse=lse)
    torch.cuda.synchronize()
    assert o2 is o and lse2 is lse


def test_split_pages_takes_int_or_auto():
    q, kp, vp, pm, t, c, cu, pl = _cpu_args()
    with pytest.raises(ValueError, match="auto"):
        cpa.chunked_prefill(q, kp, vp, pm, t, c, cu, pl, 64, split_pages="fastest")


def test_prefill_refuses_mis_shaped_tables():
    # the kernel reads tables + group * cap for every (sequence, group): a table of the wrong
    # shape is refused before any device or library call (CPU tensors reach the shape checks)
    q, kp, vp, pm, t, c, cu, pl = _cpu_args()
    for bad in (torch.zeros(2, dtype=torch.int32),              # flat
                torch.zeros(1, 2, 2, dtype=torch.int32),        # two groups for Hkv = 1
                torch.zeros(2, 1, 2, dtype=torch.int32)):       # two sequences for B = 1
        with pytest.raises(ValueError, match="tables"):
            cpa.chunked_prefill(q, kp, vp, pm, bad, c, cu, pl, 64)


def test_direct_refuses_mis_shaped_plan_counts():
    q, kp, vp, pm, t, c, cu, pl = _cpu_args()
    vd = vp.transpose(2, 3).contiguous()
    plans = torch.zeros(1, 4, 1, 2, dtype=torch.int32)
    for bad in (torch.zeros(4, dtype=torch.int32),               # [B*Hq] only: no query-block axis
                torch.zeros(1, 4, 2, dtype=torch.int32),         # two query blocks for plans of one
                torch.zeros(1, 2, 1, dtype=torch.int32)):        # two heads for Hq = 4
        with pytest.raises(ValueError, match="plan_counts"):
            cpa.chunked_prefill_direct(q, kp, vd, pm, plans, bad, cu, pl, 64)


def test_fused_checks_masks_before_the_device():
    # the fused binding checks the masks' dtype, shape and (bit-packed) block count before it
    # looks at devices, so these run on the CPU
    q, kp, vp, pm, t, c, cu, pl = _cpu_args()
    good = torch.zeros(1, 4, 1, 2, dtype=torch.uint8)
    with pytest.raises(TypeError, match="masks"):
        cpa.chunked_prefill_fused(q, kp, vp, pm, good.float(), cu, pl, 64)
    with pytest.raises(TypeError, match="masks"):
        cpa.chunked_prefill_fused(q, kp, vp, pm, good[0], cu, pl, 64)
    with pytest.raises(ValueError, match="nkvb_max"):
        cpa.chunked_prefill_fused(q, kp, vp, pm, torch.zeros(1, 4, 1, 1, dtype=torch.int64), cu, pl, 64)
    with pytest.raises(ValueError, match=r"\[B\]\[Hq\]"):
        cpa.chunked_prefill_fused(q, kp, vp, pm, torch.zeros(2, 4, 1, 2, dtype=torch.uint8), cu, pl, 64)
    with pytest.raises(ValueError, match=r"\[B\]\[Hq\]"):
        cpa.chunked_prefill_fused(q, kp, vp, pm, torch.zeros(1, 3, 1, 2, dtype=torch.uint8), cu, pl, 64)
    with pytest.raises(TypeError, match="bf16"):
        cpa.chunked_prefill_fused(q.float(), kp.float(), vp.float(), pm, good, cu, pl, 64)
    with pytest.raises(TypeError, match="CUDA"):
        cpa.chunked_prefill_fused(q, kp, vp, pm, good, cu, pl, 64)
