"""OCP FP8 E4M3 ("e4m3fn") decoding and encoding, written from the format
definition.

Test infrastructure only (see the package docstring).

Format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
field 0 encodes subnormals m/8 * 2^-6; there are no infinities and the codes
S.1111.111 are NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
FlashPrefill V2 feeds Q, K and V as e4m3 with one fp32 scale per tensor
(FlashPrefill V2, the FP8 paragraph); the oracle reads each input as
decode(code) * scale in float64.
"""
import numpy as np


def decode_e4m3fn(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    out = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, out)


def encode_e4m3fn(x) -> np.ndarray:
    """Nearest e4m3fn code of each float (ties to the even code), with
    magnitudes above the largest finite value 448 saturated to it.  Written
    from the format: the representable magnitudes are enumerated from the
    field definitions above and each input picks the closest one."""
    mags = _MAGNITUDES
    a = np.minimum(np.abs(np.asarray(x, dtype=np.float64)), 448.0)
    # index of the largest representable magnitude <= a, and the next one up
    lo = np.searchsorted(mags, a, side="right") - 1
    hi = np.minimum(lo + 1, mags.size - 1)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    # the codes of consecutive magnitudes are consecutive integers, so the
    # even mantissa is the even code
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    # the sign is kept, also for values that round to zero
    neg = np.signbit(np.asarray(x, dtype=np.float64))
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_per_tensor(x) -> tuple:
    """Online per-tensor quantisation of Q, K or V to e4m3 (FlashPrefill V2,
    the FP8 paragraph: one absmax-derived scale per tensor): with amax =
    max |x|, scale = amax / 448 (1 when amax is 0) and code = e4m3(x / scale).
    The scale and the quotient are rounded to float32, the precision the
    device takes these decisions in, so the codes are comparable bit for bit.
    Returns (codes uint8, scale as a float32 value)."""
    xf = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0.0)
    scale = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    q = (xf / scale).astype(np.float32)
    return encode_e4m3fn(q), scale


# every non-negative finite e4m3 magnitude, in code order (0 .. 448)
_MAGNITUDES = np.array([decode_e4m3fn(c) for c in range(0x7F)], dtype=np.float64)
