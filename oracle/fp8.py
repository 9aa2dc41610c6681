"""fp8 KV dequantization written out (test infrastructure; see package header).

Source: "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract
(KV blocks read in place from a paged cache).  With an fp8 cache the keys and values attention
sees are the stored e4m3 codes decoded and multiplied by the tensor's scale: v = decode(x) * scale,
taken exactly (float64).

decode(x) for the OCP e4m3 format (8 bits: sign s, 4 exponent bits e, 3 mantissa bits m,
exponent bias 7, no infinities):
  e == 15 and m == 7:  NaN
  e == 0:              (-1)^s * 2^-6 * m / 8        (subnormal; m == 0 gives a signed zero)
  otherwise:           (-1)^s * 2^(e - 7) * (1 + m / 8)
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


def dequant_e4m3(codes, scale):
    """The values an fp8 page holds for attention: decode(x) * scale, in float64."""
    return decode_e4m3(codes) * float(np.float32(scale))
