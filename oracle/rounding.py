"""Rounding of float64 values to the storage precisions the step declares.

bf16: 8 significant bits (7 stored), exponent range of fp32, round to nearest,
ties to even, gradual underflow below 2**-126, overflow to +-inf.
fp32: NumPy's own IEEE cast (round to nearest even).
"""
import numpy as np

_BF16_MAX = float.fromhex("0x1.fep127")


def round_bf16(x):
    """Nearest bf16 value of each element (ties to even), returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, ex = np.frexp(xf)                    # xf = m * 2**ex, 0.5 <= |m| < 1
    ulp_exp = np.maximum(ex - 8, -133)      # 8 significant bits; subnormal spacing 2**-133
    r = np.ldexp(np.round(np.ldexp(xf, -ulp_exp)), ulp_exp)   # np.round: half to even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def round_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, dtype):
    """Round to the storage dtype "bf16" or "f32"."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)


def bf16_bits_to_f64(bits):
    """Decode bf16 bit patterns (uint16) into float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Encode float64 values as bf16 bit patterns, rounding to nearest even."""
    r = round_bf16(x).astype(np.float32)    # exact: every bf16 value is an fp32 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def as_f64(arr, dtype):
    """Storage array (uint16 bf16 bits or float32) -> float64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float64)
