"""OCP float8 E4M3 (E4M3FN) codec -- oracle side (test infrastructure only).

The pages name the format but do not define it: whisper-blaze 0.1.8 (PyPI
page) lists "FP8 (E4M3 / E5M2)" and a ``quantise_e4m3`` call under "Direct
Kernel API"; the HF blog "Blazingly fast whisper transcriptions with
Inference Endpoints", section "Inference Stack", stores the KV cache in one
byte.  The reading taken here is the OCP 8-bit floating point E4M3 variant
(the one Ada/Hopper and gfx950 implement natively):

    bit layout  s eeee mmm, exponent bias 7
    e == 0            value = (-1)^s * m * 2^-9            (subnormals, +-0)
    e in 1..15        value = (-1)^s * (1 + m/8) * 2^(e-7)
    e == 15, m == 7   NaN (codes 0x7F and 0xFF); there is no infinity

so the largest finite magnitude is 448 (0x7E), the smallest normal 2^-6
(0x08) and the smallest subnormal 2^-9 (0x01).

Encoding rounds to nearest with ties to the even mantissa and saturates:
magnitudes above 448 become 448.  The sign bit is always the input's sign,
so -0.0 and negative values that round to zero encode as 0x80.  Non-finite
inputs are outside the contract.
"""
import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_MIN_SUBNORMAL = 2.0 ** -9


def decode_table():
    """Value of each of the 256 codes, as float64 (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 15 and m == 7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * m * 2.0 ** -9
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_TABLE = decode_table()


def decode(codes):
    """uint8 codes (any shape) -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(y):
    """float32 values (any shape) -> uint8 E4M3 codes, RNE and saturating.

    Every operation below is exact in float32 except the two intended
    round-to-nearest-even steps (``np.rint`` rounds halves to even).
    """
    y = np.asarray(y, dtype=np.float32)
    neg = np.signbit(y)
    a = np.minimum(np.abs(y), np.float32(E4M3_MAX))

    code = np.zeros(y.shape, dtype=np.int32)

    # Subnormal range (|y| < 2^-6): step 2^-9, so m = rint(a * 2^9).  A
    # result of 8 is exactly the smallest normal, whose code is 0x08.
    sub = a < np.float32(E4M3_MIN_NORMAL)
    m_sub = np.rint(a[sub] * np.float32(512.0)).astype(np.int32)
    code[sub] = m_sub

    # Normal range: a = f * 2^k with f in [0.5, 1), so the unbiased exponent
    # is k - 1 and the significand a / 2^(k-1) lies in [1, 2).
    nrm = ~sub
    f, k = np.frexp(a[nrm])
    e = k.astype(np.int32) - 1
    sig = np.ldexp(f, 1)                      # a / 2^e, exact
    m = np.rint((sig - np.float32(1.0)) * np.float32(8.0)).astype(np.int32)
    carry = m == 8                             # rounded up to the next binade
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code[nrm] = ((e + 7) << 3) | m

    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)
