"""Pins for the oracle's E4M3 codec, independent of the codec's own code.

* decode: every code against torch's float8_e4m3fn (a library reading of the
  same OCP format) and against the OCP landmark table in tests/golden;
* encode: every finite bf16 pattern and every E4M3 midpoint +-1 ulp against a
  brute-force nearest-value search with the even-mantissa tie rule, and
  against torch's own conversion after clamping to +-448.
"""
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_landmarks.txt")


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_float8_e4m3fn():
    ours = e4m3.decode_table()
    ref = _torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # signed zeros too
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_golden_landmarks():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for code_s, val_s in rows:
        code = int(code_s, 16)
        got = e4m3.decode(np.uint8(code))
        if val_s == "nan":
            assert np.isnan(got), code_s
        else:
            want = float(val_s)
            assert got == want and np.signbit(got) == np.signbit(want), (code_s, got, want)


def test_decode_structure():
    t = e4m3.decode_table()
    fin = t[~np.isnan(t)]
    assert fin.size == 254                      # 0x7f and 0xff are the only NaNs
    assert np.unique(fin).size == 253           # +0 and -0 compare equal
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)             # codes 0x00..0x7e strictly increasing
    assert np.array_equal(t[0x80:0xFF], -pos)   # sign-magnitude


def _brute_encode(vals):
    """Nearest finite E4M3 value by exhaustive search; ties -> even mantissa;
    saturate above 448; the sign bit follows the input's sign."""
    table = e4m3.decode_table()[:0x7F]          # the 127 non-negative values
    codes = np.arange(0x7F)
    vals = np.asarray(vals, dtype=np.float64)
    a = np.minimum(np.abs(vals), 448.0)
    d = np.abs(a[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    n_cand = cand.sum(axis=1)
    # unique nearest, or a tie between two neighbours: take the even code
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(n_cand[:, None] == 1, cand, even)
    assert np.all(pick.sum(axis=1) == 1)
    out = codes[np.argmax(pick, axis=1)]
    out = np.where(np.signbit(vals), out | 0x80, out)
    return out.astype(np.uint8)


def _all_finite_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


def test_encode_exhaustive_bf16_vs_brute_force():
    f = _all_finite_bf16_as_f32()
    got = e4m3.encode(f)
    want = np.concatenate([_brute_encode(c) for c in np.array_split(f, 16)])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(f[i]), int(got[i]), int(want[i])) for i in bad[:8]]


def _midpoints_and_neighbours():
    t = e4m3.decode_table()[:0x7F].astype(np.float32)
    mids = ((t[:-1].astype(np.float64) + t[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (t[:-1].astype(np.float64) + t[1:]) / 2)  # exact
    pts = np.concatenate([t, mids, [448.0, 449.0, 464.0, 1e6, 1e-30, 2.0 ** -10, 3 * 2.0 ** -11]])
    pts = pts.astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(-np.inf))
    allp = np.concatenate([pts, up, dn])
    allp = allp[allp >= 0]
    return np.concatenate([allp, -allp, np.float32([0.0, -0.0])]).astype(np.float32)


def test_encode_midpoints_and_neighbours_vs_brute_force():
    v = _midpoints_and_neighbours()
    got = e4m3.encode(v)
    want = _brute_encode(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:8]]


def test_encode_matches_torch_after_clamp():
    v = np.concatenate([_all_finite_bf16_as_f32(), _midpoints_and_neighbours()])
    clamped = np.clip(v, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3.encode(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(ref[i])) for i in bad[:8]]


@pytest.mark.parametrize("x,code", [(448.0, 0x7E), (1e9, 0x7E), (-1e9, 0xFE), (-0.0, 0x80),
                                    (-1e-30, 0x80), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
                                    (3 * 2.0 ** -11, 0x01),
                                    (0.0146484375, 0x08)])
def test_encode_special_cases(x, code):
    # 2^-10 is the tie between 0 and 2^-9: even mantissa -> 0.  3*2^-10 is the
    # tie between 1*2^-9 and 2*2^-9: even -> 0x02; 3*2^-11 (0.75 * 2^-9) is
    # nearest to 2^-9.  0.0146484375 is the tie
    # between the largest subnormal 7*2^-9 and 2^-6: even -> 0x08.
    assert int(e4m3.encode(np.float32(x))) == code
