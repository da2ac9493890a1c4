"""Pins for the oracle's E5M2 codec, independent of the codec's own code.

* decode: every code against torch's float8_e5m2 (a library reading of the
  same OCP format), against IEEE binary16 with the code as its upper byte
  (numpy float16; the OCP E5M2 layout is binary16 cut to two mantissa bits),
  and against the OCP landmark table in tests/golden;
* encode: every finite bf16 pattern and every E5M2 midpoint +-1 ulp against a
  brute-force nearest-value search with the even-mantissa tie rule; every
  finite binary16 value against round-to-nearest-even on its bit pattern;
  and against torch's own conversion after clamping to +-57344.
"""
import os

import numpy as np
import pytest
import torch

from oracle import e5m2
from tests.test_oracle_e4m3 import _all_finite_bf16_as_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e5m2_landmarks.txt")


def _same(a, b):
    """Equal as values, NaN equal to NaN, signed zeros and infinities kept."""
    a, b = np.asarray(a), np.asarray(b)
    nan = np.isnan(a)
    return (np.array_equal(nan, np.isnan(b)) and np.array_equal(a[~nan], b[~nan])
            and np.array_equal(np.signbit(a[~nan]), np.signbit(b[~nan])))


def test_decode_matches_torch_float8_e5m2():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    assert _same(e5m2.decode_table(), ref)


def test_decode_matches_binary16_upper_byte():
    half = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    assert _same(e5m2.decode_table(), half)


def test_decode_golden_landmarks():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 15
    for code_s, val_s in rows:
        got = e5m2.decode(np.uint8(int(code_s, 16)))
        assert _same(np.float64([got]), np.float64([float(val_s)])), (code_s, got, val_s)


def test_decode_structure():
    t = e5m2.decode_table()
    assert np.sum(np.isnan(t)) == 6 and np.sum(np.isinf(t)) == 2
    pos = t[:0x7C]                                # the finite non-negative codes
    assert np.all(np.diff(pos) > 0)
    assert _same(t[0x80:0xFC], -pos)


def _brute_encode(vals):
    """Nearest finite E5M2 value by exhaustive search; ties -> even mantissa;
    saturate above 57344; the sign bit follows the input's sign."""
    table = e5m2.decode_table()[:0x7C]
    codes = np.arange(0x7C)
    vals = np.asarray(vals, dtype=np.float64)
    a = np.minimum(np.abs(vals), e5m2.E5M2_MAX)
    d = np.abs(a[:, None] - table[None, :])
    cand = d == d.min(axis=1, keepdims=True)
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(cand.sum(axis=1)[:, None] == 1, cand, even)
    assert np.all(pick.sum(axis=1) == 1)
    out = codes[np.argmax(pick, axis=1)]
    return np.where(np.signbit(vals), out | 0x80, out).astype(np.uint8)


def test_encode_exhaustive_bf16_vs_brute_force():
    f = _all_finite_bf16_as_f32()
    got = e5m2.encode(f)
    want = np.concatenate([_brute_encode(c) for c in np.array_split(f, 16)])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(f[i]), int(got[i]), int(want[i])) for i in bad[:8]]


def test_encode_binary16_by_bit_rounding():
    # a finite binary16 pattern h rounds to E5M2 by dropping its low 8 bits,
    # nearest-even: add 0x7f plus the lowest kept bit, then shift; a carry
    # into the infinity pattern saturates to the largest finite code
    h = np.arange(65536, dtype=np.uint32)
    v = h.astype(np.uint16).view(np.float16)
    fin = np.isfinite(v)
    h, v = h[fin], v[fin].astype(np.float32)
    mag = h & 0x7FFF
    r = (mag + 0x7F + ((mag >> 8) & 1)) >> 8
    r = np.minimum(r, 0x7B)
    want = (r | ((h >> 8) & 0x80)).astype(np.uint8)
    got = e5m2.encode(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:8]]


def _midpoints_and_neighbours():
    t = e5m2.decode_table()[:0x7C].astype(np.float32)
    mids = ((t[:-1].astype(np.float64) + t[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (t[:-1].astype(np.float64) + t[1:]) / 2)
    pts = np.concatenate([t, mids, [57344.0, 57345.0, 61440.0, 1e9, 1e-30, 2.0 ** -17,
                                    3 * 2.0 ** -18]]).astype(np.float32)
    allp = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)),
                           np.nextafter(pts, np.float32(-np.inf))])
    allp = allp[allp >= 0]
    return np.concatenate([allp, -allp, np.float32([0.0, -0.0])]).astype(np.float32)


def test_encode_midpoints_and_neighbours_vs_brute_force():
    v = _midpoints_and_neighbours()
    got = e5m2.encode(v)
    want = _brute_encode(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:8]]


def test_encode_matches_torch_after_clamp():
    v = np.concatenate([_all_finite_bf16_as_f32(), _midpoints_and_neighbours()])
    clamped = np.clip(v, -e5m2.E5M2_MAX, e5m2.E5M2_MAX).astype(np.float32)
    ref = torch.from_numpy(clamped).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = e5m2.encode(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(ref[i])) for i in bad[:8]]


@pytest.mark.parametrize("x,code", [(57344.0, 0x7B), (61440.0, 0x7B), (1e9, 0x7B), (-1e9, 0xFB),
                                    (-0.0, 0x80), (2.0 ** -17, 0x00), (3 * 2.0 ** -17, 0x02),
                                    (1.125, 0x3C), (1.375, 0x3E), (7 * 2.0 ** -17, 0x04)])
def test_encode_special_cases(x, code):
    # 61440 is the midpoint between 57344 and the infinity pattern: saturates.
    # 2^-17 ties 0 and 2^-16 -> even 0; 3*2^-17 ties 1 and 2 (x 2^-16) -> 2;
    # 1.125 ties 1.0 and 1.25 -> 1.0 (even); 1.375 ties 1.25 and 1.5 -> 1.5;
    # 7*2^-17 ties the largest subnormal 3*2^-16 and 2^-14 -> 0x04 (even).
    assert int(e5m2.encode(np.float32(x))) == code
