"""Storage formats, decoded independently of the HIP library (test infrastructure only).

The indexer's inputs arrive as raw storage: IEEE float32, bfloat16 (the upper
16 bits of a float32) or OCP FP8 E4M3 ("e4m3fn": 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN,
largest finite magnitude 448) with one float32 scale per token.  Every
function here maps those bits to exact float64 values; nothing is rounded
except by ``f64_to_bf16_bits_rne``, which is the one place the oracle models
a storage rounding (the proxy query's format, see ``indexer.round_proxy``).
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> exact float64 values.

    A bfloat16 is the high half of an IEEE binary32, so widening the pattern
    by 16 zero bits gives the same number as a float32.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_bits_to_f64(bits):
    """OCP FP8 E4M3 bit patterns (uint8) -> exact float64 values (NaN for S.1111.111)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * np.exp2(1.0 - 7.0)
    val = np.where(e == 0, subnormal, normal)
    val = np.where((e == 0xF) & ((b & 0x7) == 0x7), np.nan, val)
    return sign * val


def f64_to_bf16_bits_rne(x):
    """float64 -> nearest bfloat16 (ties to even), returned as uint16 bit patterns.

    Rounds once, directly from float64: the quantum of a value whose leading
    bit is 2^(e-1) is 2^(e-8) (8 significant bits), floored at the subnormal
    quantum 2^-133.  ``numpy.round`` rounds halves to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    quantum = np.exp2(np.maximum(e.astype(np.float64) - 8.0, -133.0))
    r = np.round(x / quantum) * quantum
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def real_values(raw, fmt, scale=None):
    """Decode raw storage to float64 and apply the per-token scale.

    raw   : float32 array (fmt "f32"), uint16 bit patterns ("bf16") or uint8
            bit patterns ("fp8"); the leading axes are (sequence, token), the
            trailing axes are the token's payload (heads and/or dimension).
    scale : float32 [sequence, token] for "fp8" (one scale per token, shared
            by all of the token's payload), None otherwise.
    """
    if fmt == "f32":
        vals = np.asarray(raw, dtype=np.float32).astype(np.float64)
    elif fmt == "bf16":
        vals = bf16_bits_to_f64(raw)
    elif fmt == "fp8":
        vals = e4m3fn_bits_to_f64(raw)
    else:
        raise ValueError(f"unknown storage format {fmt!r}")
    if fmt == "fp8":
        if scale is None:
            raise ValueError("fp8 storage needs a per-token scale")
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        vals = vals * s.reshape(s.shape + (1,) * (vals.ndim - s.ndim))
    elif scale is not None:
        raise ValueError("a scale is only defined for fp8 storage")
    return vals
