"""Pins for the oracle's E5M2 quantization and its dequantise (both formats).

* E5M2 quantize: exhaustive bf16 at several scales against an fp64 quotient
  plus nearest-value search; the amax element maps to +-57344; the round-trip
  error is within half an E5M2 ulp; a pure-Python brute force of the fill;
* bf16 rounding: every bf16 value, their midpoints and neighbours, and random
  fp32 patterns against torch's float32 -> bfloat16 conversion;
* dequantise: every code at several scales against torch (float8 view, fp32
  multiply, bfloat16 conversion); with a power-of-two scale the result is
  the exact value rounded once; the inverse read of a fill puts each valid
  position back within the round-trip bound and leaves the rest untouched.
"""
import math

import numpy as np
import pytest
import torch

from oracle import e4m3, e5m2, quant
from tests.test_oracle_e4m3 import _all_finite_bf16_as_f32
from tests.test_oracle_e5m2 import _brute_encode as _brute_e5m2
from tests.test_oracle_quant import _py_round_even, _sample

SCALES = [1.0, 2.0 ** -3, np.float32(4.25 / 57344), np.float32(93.0 / 57344), np.float32(2.0 ** -20 / 3)]
TORCH_FMT = {quant.E4M3: torch.float8_e4m3fn, quant.E5M2: torch.float8_e5m2}


@pytest.mark.parametrize("s", SCALES)
def test_quantize_e5m2_exhaustive_bf16(s):
    s = np.float32(s)
    x = _all_finite_bf16_as_f32().reshape(1, -1, 1, 1)
    got = quant.quantize(x, np.float32([s]), quant.PER_TENSOR, quant.E5M2).ravel()
    # the fp64 quotient of an 8-bit and a 24-bit significand rounds to the
    # IEEE fp32 quotient when rounded once more to fp32
    with np.errstate(over="ignore"):           # beyond fp32 saturates in the encode
        y = (x.ravel().astype(np.float64) / np.float64(s)).astype(np.float32)
    want = np.concatenate([_brute_e5m2(c) for c in np.array_split(y, 16)])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x.ravel()[i]), int(got[i]), int(want[i])) for i in bad[:8]]


def test_e5m2_amax_element_and_round_trip_bound():
    x = _sample((2, 64, 3, 64))
    lens = np.array([64, 40])
    for gran in (quant.PER_TENSOR, quant.PER_HEAD):
        amax = quant.group_amax(x, lens, gran)
        s = quant.scales_from_amax(amax, quant.E5M2)
        assert np.array_equal(s, (amax / np.float32(57344.0)).astype(np.float32))
        c = quant.quantize(x, s, gran, quant.E5M2)
        mask = quant.valid_mask(2, 64, lens)
        for g in range(amax.size):
            sub = x[mask] if gran == quant.PER_TENSOR else x[mask][:, g, :]
            cs = c[mask] if gran == quant.PER_TENSOR else c[mask][:, g, :]
            at = np.abs(sub) == amax[g]
            assert at.any() and np.all((cs[at] & 0x7F) == 0x7B)
        back = quant.dequantize(c, s, gran, head_axis=2, fmt=quant.E5M2)
        sb = np.broadcast_to(s.reshape(1, 1, -1, 1) if gran else s.reshape(1, 1, 1, 1), x.shape)
        y = np.abs(x / sb)
        err = np.abs(back - x)
        normal = y >= 2.0 ** -14
        # half an E5M2 ulp: 2^-3 relative for normals, 2^-17 * scale below
        assert np.all(err[normal] <= 2.0 ** -3 * np.abs(x[normal]) * (1 + 2.0 ** -20))
        assert np.all(err[~normal] <= 2.0 ** -17 * sb[~normal] * (1 + 2.0 ** -20))


def test_e5m2_fill_brute_force_pure_python():
    """The E5M2 fill with Python scalars: binade by doubling/halving, two
    mantissa bits, the step count rounded half-to-even."""
    x = _sample((2, 5, 3, 4))
    lens, dst, L = [5, 3], [0, 2], 8
    for gran in (quant.PER_TENSOR, quant.PER_HEAD):
        cache = np.zeros((2, 3, L, 4), dtype=np.uint8)
        s_or = quant.quantize_kv(x, lens, dst, cache, gran, quant.E5M2)
        for b in range(2):
            for t in range(lens[b]):
                for h in range(3):
                    for d in range(4):
                        sc = s_or[0 if gran == quant.PER_TENSOR else h]
                        y = float(np.float32(np.float32(x[b, t, h, d]) / sc))
                        a = min(abs(y), 57344.0)
                        e = 0
                        while a >= 2.0 ** (e + 1) and e < 15:
                            e += 1
                        while a < 2.0 ** e and e > -14:
                            e -= 1
                        n = _py_round_even(a / 2.0 ** (e - 2))    # 2 mantissa bits
                        if e == -14 and a < 2.0 ** -14:
                            code = n                            # subnormal, step 2^-16
                        else:
                            if n == 8:
                                e, n = e + 1, 4
                            code = ((e + 15) << 2) | (n - 4)
                        if math.copysign(1.0, y) < 0:
                            code |= 0x80
                        assert cache[b, h, dst[b] + t, d] == code, (b, t, h, d, y, code)


def _torch_bf16_bits(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_bf16_rounding_matches_torch():
    f = _all_finite_bf16_as_f32()
    nxt = (f.view(np.uint32) + 0x10000).view(np.float32)
    mids = np.where(np.isfinite(nxt), (f.view(np.uint32) + 0x8000).view(np.float32), f)
    pts = np.concatenate([f, mids, np.nextafter(mids, np.float32(np.inf)),
                          np.nextafter(mids, np.float32(-np.inf))]).astype(np.float32)
    rnd = np.random.default_rng(0).integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64)
    r = rnd.astype(np.uint32).view(np.float32)
    pts = np.concatenate([pts, r[np.isfinite(r)]])
    got = quant.bf16_rne_bits(pts)
    want = _torch_bf16_bits(pts)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(pts[i]), int(got[i]), int(want[i])) for i in bad[:8]]


# the last two give fp32 subnormal products and products near the fp32 top
DQ_SCALES = [1.0, 0.125, 1.0 / 448, 93.0 / 57344, 3.0e-3, float.fromhex("0x1.8p-120"),
             float.fromhex("0x1.fffffep100")]


@pytest.mark.parametrize("fmt", [quant.E4M3, quant.E5M2])
@pytest.mark.parametrize("s", DQ_SCALES)
def test_dequantise_every_code_vs_torch(fmt, s):
    codes = np.arange(256, dtype=np.uint8).reshape(1, 1, 256, 1)
    s = np.float32(s)
    got = quant.dequantise_bf16(codes, np.float32([s]), quant.PER_TENSOR, 1, fmt).ravel()
    v = torch.from_numpy(codes.ravel().copy()).view(TORCH_FMT[fmt]).to(torch.float32)
    want = (v * torch.tensor(s, dtype=torch.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)
    gf = got.astype(np.uint32) << 16
    wf = want.astype(np.uint32) << 16
    gv, wv = gf.view(np.float32), wf.view(np.float32)
    both_nan = np.isnan(gv) & np.isnan(wv)
    bad = np.nonzero((got != want) & ~both_nan)[0]
    assert bad.size == 0, [(int(i), int(got[i]), int(want[i])) for i in bad[:8]]


@pytest.mark.parametrize("fmt,table", [(quant.E4M3, e4m3.decode_table()), (quant.E5M2, e5m2.decode_table())])
def test_dequantise_power_of_two_scale_is_one_rounding(fmt, table):
    # with s = 2^k the fp32 product is exact, so the bf16 result must be the
    # exact value rounded once to nearest even: for these formats every code
    # value already fits bf16's 8-bit significand, so it is the value itself
    codes = np.arange(256, dtype=np.uint8).reshape(1, 1, -1, 1)
    fin = np.isfinite(table)
    for k in (-3, 0, 5):
        got = quant.dequantise_bf16(codes, np.float32([2.0 ** k]), quant.PER_TENSOR, 1, fmt).ravel()
        val = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.array_equal(val[fin], table[fin] * 2.0 ** k)
        assert np.array_equal(np.signbit(val[fin]), np.signbit(table[fin]))


@pytest.mark.parametrize("fmt", [quant.E4M3, quant.E5M2])
def test_unfill_inverts_fill(fmt):
    x = _sample((3, 9, 4, 64))
    lens = np.array([9, 5, 0])
    half_ulp = {quant.E4M3: (2.0 ** -4, 2.0 ** -6, 2.0 ** -10),
                quant.E5M2: (2.0 ** -3, 2.0 ** -14, 2.0 ** -17)}[fmt]
    for gran in (quant.PER_TENSOR, quant.PER_HEAD):
        cache = np.zeros((3, 4, 12, 64), dtype=np.uint8)
        s = quant.quantize_kv(x, lens, np.zeros(3, np.int32), cache, gran, fmt)
        out = quant.unfill_cache(cache, lens, s, gran, 9, fmt)
        sb = s.reshape(1, -1, 1) if gran else s.reshape(1, 1, 1)
        for b in range(3):
            assert np.all(out[b, lens[b]:] == 0xFFFF)
            if lens[b] == 0:
                continue
            back = (out[b, :lens[b]].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            xb = x[b, :lens[b]].astype(np.float64)
            y = np.abs(xb / sb)
            sbb = np.broadcast_to(sb, xb.shape)
            # fp8 half ulp, then the bf16 store's half ulp (2^-9 relative)
            lim = np.where(y >= half_ulp[1], half_ulp[0] * np.abs(xb), half_ulp[2] * sbb)
            lim = lim * (1 + 2.0 ** -20) + 2.0 ** -8 * (np.abs(xb) + lim)
            assert np.all(np.abs(back - xb) <= lim)
