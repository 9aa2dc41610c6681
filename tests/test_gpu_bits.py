"""GPU parity of the table build from bit-packed masks (cpa_build_block_tables_bits): tables and
counts bit-exact against the oracle on the unpacked masks, and equal to the byte-mask build."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_reduce_amd as cpa
from workloads import make_config, make_workload
from workloads.configs import mask_all, mask_bernoulli, pack_mask_bits

from _gpu import gpu_tables, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def bern(p, local=1):
    return lambda rng, *a: mask_bernoulli(rng, *a, p=p, local=local)


SMALL = {
    "g4_noise": dict(prefix_len=[448, 64], chunk_len=[192, 256], Hq=8, Hkv=2, mask_fn=bern(0.1), noncausal_noise=0.3),
    "partial_word_70": dict(prefix_len=[64 * 66], chunk_len=[256], Hq=8, Hkv=2, mask_fn=bern(0.03)),
    "g1_varlen": dict(prefix_len=[0, 640, 1280], chunk_len=[320, 192, 64], Hq=4, Hkv=4, mask_fn=bern(0.2)),
    "g8": dict(prefix_len=[512], chunk_len=[256], Hq=16, Hkv=2, mask_fn=bern(0.1)),
    "all_ones": dict(prefix_len=[256, 0], chunk_len=[192, 128], Hq=8, Hkv=2, mask_fn=lambda rng, *a: mask_all(rng, *a, value=1)),
    "all_zero": dict(prefix_len=[256], chunk_len=[128], Hq=8, Hkv=2, mask_fn=lambda rng, *a: mask_all(rng, *a, value=0)),
    "zero_len_chunk": dict(prefix_len=[128, 256], chunk_len=[0, 128], Hq=8, Hkv=2, mask_fn=bern(0.3)),
}


def check(w, extra_words=0, seed=0):
    bits = pack_mask_bits(w.masks)
    if extra_words:   # wider rows with garbage past the last block: ignored
        rng = np.random.default_rng(seed)
        pad = rng.integers(0, 2 ** 63, size=bits.shape[:3] + (extra_words,), dtype=np.int64).view(np.uint64)
        bits = np.concatenate([bits, pad], axis=-1)
    if w.nkvb_max % 64:   # garbage in the unused bits of the last word: ignored
        hi = np.uint64(((1 << 64) - 1) ^ ((1 << (w.nkvb_max % 64)) - 1))
        bits[..., (w.nkvb_max - 1) // 64] |= hi
    dv = upload(w)
    tb = torch.from_numpy(np.ascontiguousarray(bits).view(np.int64)).cuda()
    t1, c1 = cpa.build_block_tables_bits(tb, w.nkvb_max, dv["pb"], dv["cb"], w.Hkv)
    t0, c0 = gpu_tables(dv, w)
    T, C = oracle.block_union_tables_bits(bits, w.nkvb_max, w.prefix_blocks, w.chunk_blocks, w.Hkv)
    assert np.array_equal(t1.cpu().numpy(), T) and np.array_equal(c1.cpu().numpy(), C)
    assert torch.equal(t1, t0) and torch.equal(c1, c0)


@pytest.mark.parametrize("extra", [0, 3])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_bits_small(name, extra):
    kw = dict(SMALL[name])
    w = make_workload(name, kw.pop("prefix_len"), kw.pop("chunk_len"), kw.pop("Hq"), kw.pop("Hkv"), 64, "bf16",
                      kw.pop("mask_fn"), 13, **kw)
    check(w, extra_words=extra)


@pytest.mark.parametrize("name", ["c3_128k_last_chunk", "c5b_varlen_independent", "c2_32k_bf16"])
def test_bits_full_size(name):
    print(f"\n[case] bit-packed tables {name}", flush=True)
    check(make_config(name))
