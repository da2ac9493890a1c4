"""OCP float8 E5M2 codec -- oracle side (test infrastructure only).

whisper-blaze 0.1.8 (PyPI page) lists "FP8 (E4M3 / E5M2)" among its
features; the pages define neither format.  The reading taken here is the
OCP 8-bit floating point E5M2 variant (the one gfx950 converts natively):

    bit layout  s eeeee mm, exponent bias 15 (the upper byte of an IEEE
    binary16 value)
    e == 0            value = (-1)^s * m * 2^-16           (subnormals, +-0)
    e in 1..30        value = (-1)^s * (1 + m/4) * 2^(e-15)
    e == 31, m == 0   +-infinity;  e == 31, m != 0  NaN

so the largest finite magnitude is 57344 (0x7B), the smallest normal 2^-14
(0x04) and the smallest subnormal 2^-16 (0x01).

Encoding rounds to nearest with ties to the even mantissa and saturates:
magnitudes above 57344 become 57344 (never infinity).  The sign bit is the
input's sign, so -0.0 and negative values that round to zero encode as 0x80.
Non-finite inputs are outside the contract.
"""
import numpy as np

E5M2_MAX = 57344.0
E5M2_MIN_NORMAL = 2.0 ** -14
E5M2_MIN_SUBNORMAL = 2.0 ** -16


def decode_table():
    """Value of each of the 256 codes as float64 (+-inf and NaN included)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 2) & 0x1F
        m = code & 0x3
        if e == 31:
            out[code] = sign * np.inf if m == 0 else np.nan
        elif e == 0:
            out[code] = sign * m * 2.0 ** -16
        else:
            out[code] = sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)
    return out


_TABLE = decode_table()


def decode(codes):
    """uint8 codes (any shape) -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(y):
    """float32 values (any shape) -> uint8 E5M2 codes, RNE and saturating.

    The magnitude is split into a binade and a position inside it; the two
    mantissa bits are the position rounded half-to-even (``np.rint``), and a
    round-up out of the binade moves to the next exponent.  Every step is
    exact in float32 except that one rounding.
    """
    y = np.asarray(y, dtype=np.float32)
    neg = np.signbit(y)
    a = np.minimum(np.abs(y), np.float32(E5M2_MAX))
    code = np.zeros(y.shape, dtype=np.int32)

    # below the smallest normal the spacing is 2^-16 everywhere; a result of
    # 4 is the smallest normal itself, code 0x04
    sub = a < np.float32(E5M2_MIN_NORMAL)
    code[sub] = np.rint(a[sub] * np.float32(65536.0)).astype(np.int32)

    nrm = ~sub
    f, k = np.frexp(a[nrm])                    # a = f * 2^k, f in [0.5, 1)
    e = k.astype(np.int32) - 1                 # a in [2^e, 2^(e+1))
    frac = np.ldexp(f, 1) - np.float32(1.0)    # position in the binade, [0, 1)
    m = np.rint(frac * np.float32(4.0)).astype(np.int32)
    up = m == 4
    e = np.where(up, e + 1, e)
    m = np.where(up, 0, m)
    code[nrm] = ((e + 15) << 2) | m

    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)
