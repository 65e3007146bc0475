"""Exact bf16 decoding and single-step fp64 -> bf16 rounding (oracle side).

bf16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent bits,
7 stored significand bits.  Decoding is exact in fp64.  Rounding from fp64 is
done once, to nearest with ties to even, directly on the fp64 value (not via
an intermediate fp32, which could round twice).
"""
import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    ax = np.abs(x)
    finite = np.isfinite(x)
    normal = finite & (ax >= 2.0 ** -126)
    # normal range: 8 significant bits.  frexp gives m in [0.5, 1), so m * 2^8
    # holds the 8 kept bits left of the point; rint rounds half to even.
    m, e = np.frexp(x[normal])
    out[normal] = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    # subnormal range: fixed spacing 2^-133
    sub = finite & ~normal
    out[sub] = np.ldexp(np.rint(np.ldexp(x[sub], 133)), -133)
    out[~finite] = x[~finite]
    over = np.abs(out) > BF16_MAX
    out[over] = np.copysign(np.inf, out[over])
    f32 = out.astype(np.float32)            # exact: every bf16 value is an fp32 value
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    bits[np.isnan(x)] = 0x7FC0
    return bits


def round_to_bf16(x) -> np.ndarray:
    """fp64 -> nearest bf16 value, returned as fp64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


def decode(arr, dtype: str) -> np.ndarray:
    """Inputs as the device sees them, widened exactly to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)
