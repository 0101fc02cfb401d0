"""FP8 E4M3 cache values, decoded exactly to fp64.  Test infrastructure only
(see the package docstring).

The pages give no storage format or scale convention for an 8-bit KV cache;
they name an FP8 cache as half the bf16 bytes ("Long context (engineering
100k+ tokens)", section 1, why long context is hard; and its common
pitfalls) and a quantized cache as fewer bytes per token ("Long-context
models", "Memory grows even with efficient attention").  The reading adopted: the OCP 8-bit floating-point format E4M3
(1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
holds subnormals m/8 * 2^-6; no infinities; S.1111.111 is NaN; largest
finite value 448) and one fp32 scale per KV head, separately for K and V:
the cached value of element x is decode(byte) * scale[head].
"""

import numpy as np


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact value of each E4M3 byte (uint8 array-like) as fp64; NaN codes
    (0x7F, 0xFF) give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    subnormal = sign * (man / 8.0) * 2.0 ** -6
    out = np.where(exp == 0, subnormal, normal)
    return np.where((exp == 0xF) & ((c & 0x7) == 0x7), np.nan, out)


def dequantize_cache(codes, scale) -> np.ndarray:
    """Cache [B, L, Hkv, D] of E4M3 bytes with per-KV-head scales [Hkv] ->
    fp64 values."""
    vals = e4m3_to_f64(codes)
    return vals * np.asarray(scale, dtype=np.float64)[None, None, :, None]
