"""OCP FP8 E4M3 ("e4m3fn") decoding, written from the format definition.

Test infrastructure only (see the package docstring).

Format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
field 0 encodes subnormals m/8 * 2^-6; there are no infinities and the codes
S.1111.111 are NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
FlashPrefill V2 feeds Q, K and V as e4m3 with one fp32 scale per tensor
(FlashPrefill V2, Sec. 3.3 FP8 paragraph); the oracle reads each input as
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
