"""fp8 KV dequantization written out (test infrastructure; see package header).

Source: "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract
(KV blocks read in place from a paged cache).  With an fp8 cache the values attention sees are
the stored e4m3 codes dequantized: v = bf16(fp32(decode(x)) * fp32(scale)).

decode(x) for the OCP e4m3 format (8 bits: sign s, 4 exponent bits e, 3 mantissa bits m,
exponent bias 7, no infinities):
  e == 15 and m == 7:  NaN
  e == 0:              (-1)^s * 2^-6 * m / 8        (subnormal; m == 0 gives a signed zero)
  otherwise:           (-1)^s * 2^(e - 7) * (1 + m / 8)
bf16(y) rounds a float32 to the nearest bfloat16, ties to even (NaN stays NaN).
"""
import numpy as np


def decode_e4m3(codes):
    """uint8 codes (any shape) -> float64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = s * np.ldexp(1.0 + m / 8.0, e - 7)
    sub = s * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, out)


def round_bf16(x):
    """float32 values -> the nearest bfloat16 values (ties to even), returned as float32."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(f), np.float32(np.nan), out)


def dequant_e4m3(codes, scale):
    """The values an fp8 page holds for attention: bf16(fp32(decode(x)) * fp32(scale))."""
    y = decode_e4m3(codes).astype(np.float32) * np.float32(scale)
    return round_bf16(y)
