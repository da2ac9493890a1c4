"""Pins for the oracle's dynamic KV quantization.

Checked against what the definition fixes, not against its own code:
exhaustive bf16 inputs at several scales versus an independent fp64-quotient
plus nearest-value search; the invariants (amax element -> +-448, odd
symmetry, monotonicity, round-trip error bound, amax = 0, padding excluded,
per-tensor amax = max of per-head amax); and a pure-Python brute force of the
whole fill on a tiny ragged batch.
"""
import math

import numpy as np
import pytest

from oracle import e4m3, quant
from tests.test_oracle_e4m3 import _all_finite_bf16_as_f32, _brute_encode

SCALES = [1.0, 2.0 ** -3, np.float32(4.25 / 448), np.float32(93.0 / 448), np.float32(2.0 ** -20 / 3)]


@pytest.mark.parametrize("s", SCALES)
def test_quantize_exhaustive_bf16(s):
    s = np.float32(s)
    x = _all_finite_bf16_as_f32().reshape(1, -1, 1, 1)
    got = quant.quantize(x, np.float32([s]), quant.PER_TENSOR).ravel()
    # The correctly rounded fp32 quotient, computed another way: the fp64
    # quotient of an 8-bit and a 24-bit significand is never within an fp64
    # ulp of an fp32 rounding boundary unless exactly on it, so rounding it
    # once more to fp32 gives the IEEE fp32 result.
    y = (x.ravel().astype(np.float64) / np.float64(s)).astype(np.float32)
    want = np.concatenate([_brute_encode(c) for c in np.array_split(y, 16)])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x.ravel()[i]), int(got[i]), int(want[i])) for i in bad[:8]]


def _bf16(a):
    import torch
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def _sample(shape, seed=0, outliers=True):
    g = np.random.default_rng(seed)
    x = g.standard_normal(shape).astype(np.float32)
    if outliers:
        x = np.where(g.random(shape) < 0.01, x * 20, x)
    return _bf16(x)


def test_amax_element_hits_448_and_symmetry_and_monotone():
    x = _sample((3, 17, 4, 64))
    lens = np.array([17, 9, 1])
    for gran in (quant.PER_TENSOR, quant.PER_HEAD):
        amax = quant.group_amax(x, lens, gran)
        s = quant.scales_from_amax(amax)
        c = quant.quantize(x, s, gran)
        cn = quant.quantize(-x, s, gran)
        assert np.array_equal(cn, c ^ 0x80)
        # the element attaining a group's amax maps to +-448
        mask = quant.valid_mask(3, 17, lens)
        for g in range(amax.size):
            sub = x[mask] if gran == quant.PER_TENSOR else x[mask][:, g, :]
            cs = c[mask] if gran == quant.PER_TENSOR else c[mask][:, g, :]
            at = np.abs(sub) == amax[g]
            assert at.any()
            assert np.all((cs[at] & 0x7F) == 0x7E)
        # monotone: a larger input never gets a smaller decoded value
        flat = x.reshape(-1, 4, 64)[:, 0, :].ravel()
        order = np.argsort(flat, kind="stable")
        dec = e4m3.decode(quant.quantize(flat[order].reshape(1, -1, 1, 1), s[:1], quant.PER_TENSOR)).ravel()
        assert np.all(np.diff(dec) >= 0)


def test_round_trip_error_bound():
    x = _sample((2, 64, 3, 64))
    lens = np.array([64, 40])
    for gran in (quant.PER_TENSOR, quant.PER_HEAD):
        s = quant.scales_from_amax(quant.group_amax(x, lens, gran))
        c = quant.quantize(x, s, gran)
        back = quant.dequantize(c, s, gran, head_axis=2)
        sb = np.broadcast_to(s.reshape(1, 1, -1, 1) if gran else s.reshape(1, 1, 1, 1), x.shape)
        y = np.abs(x / sb)
        err = np.abs(back - x)
        normal = y >= 2.0 ** -6
        # half an E4M3 ulp: 2^-4 relative for normals, 2^-10 * scale for
        # subnormals; the fp32 quotient adds at most 2^-24 relative
        assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 2.0 ** -20))
        assert np.all(err[~normal] <= 2.0 ** -10 * sb[~normal] * (1 + 2.0 ** -20))


def test_amax_zero_gives_unit_scale_and_zero_codes():
    x = np.zeros((2, 5, 3, 64), dtype=np.float32)
    x[1, 2, 1, 7] = -0.0
    x[0, 1, 2, :] = -0.0
    lens = np.array([5, 5])
    for gran in (quant.PER_TENSOR, quant.PER_HEAD):
        s = quant.scales_from_amax(quant.group_amax(x, lens, gran))
        assert np.all(s == 1.0)
        c = quant.quantize(x, s, gran)
        assert np.array_equal(c, np.where(np.signbit(x), 0x80, 0x00).astype(np.uint8))


def test_padding_excluded_and_untouched():
    x = _sample((3, 11, 2, 64), outliers=False)
    lens = np.array([11, 4, 0])
    xp = x.copy()
    for b in range(3):
        xp[b, lens[b]:] = 1000.0          # garbage in the padding
    for gran in (quant.PER_TENSOR, quant.PER_HEAD):
        assert np.array_equal(quant.group_amax(x, lens, gran), quant.group_amax(xp, lens, gran))
        cache = np.full((3, 2, 16, 64), 0x5A, dtype=np.uint8)
        dst = np.array([0, 3, 7])
        s = quant.quantize_kv(xp, lens, dst, cache, gran)
        codes = quant.quantize(xp, s, gran)
        for b in range(3):
            for t in range(16):
                if dst[b] <= t < dst[b] + lens[b]:
                    assert np.array_equal(cache[b, :, t], codes[b, t - dst[b]])
                else:
                    assert np.all(cache[b, :, t] == 0x5A), (b, t)
        assert s.dtype == np.float32


def test_per_tensor_amax_is_max_of_per_head():
    x = _sample((4, 13, 5, 64))
    lens = np.array([13, 2, 7, 1])
    ph = quant.group_amax(x, lens, quant.PER_HEAD)
    pt = quant.group_amax(x, lens, quant.PER_TENSOR)
    assert pt[0] == ph.max()


def _py_round_even(v):
    f = math.floor(v)
    r = v - f
    if r > 0.5 or (r == 0.5 and f % 2 == 1):
        f += 1
    return int(f)


def test_fill_brute_force_pure_python():
    """The whole dynamic fill, written out with Python scalars on a tiny batch.

    Encode here is a separate derivation: find the binade by repeated
    doubling/halving, then round the step count half-to-even.
    """
    x = _sample((2, 5, 3, 4))
    lens = [5, 3]
    dst = [0, 2]
    L = 8
    for gran in (quant.PER_TENSOR, quant.PER_HEAD):
        cache = np.zeros((2, 3, L, 4), dtype=np.uint8)
        s_or = quant.quantize_kv(x, lens, dst, cache, gran)
        # brute force
        groups = [0] if gran == quant.PER_TENSOR else [0, 1, 2]
        amax = {g: 0.0 for g in groups}
        for b in range(2):
            for t in range(lens[b]):
                for h in range(3):
                    for d in range(4):
                        g = 0 if gran == quant.PER_TENSOR else h
                        amax[g] = max(amax[g], abs(float(x[b, t, h, d])))
        scale = {g: (np.float32(1.0) if amax[g] == 0 else np.float32(np.float32(amax[g]) / np.float32(448.0)))
                 for g in groups}
        assert [float(scale[g]) for g in groups] == [float(v) for v in s_or]
        for b in range(2):
            for t in range(lens[b]):
                for h in range(3):
                    for d in range(4):
                        g = 0 if gran == quant.PER_TENSOR else h
                        y = float(np.float32(np.float32(x[b, t, h, d]) / scale[g]))
                        a = min(abs(y), 448.0)
                        e = 0
                        while a >= 2.0 ** (e + 1) and e < 8:
                            e += 1
                        while a < 2.0 ** e and e > -6:
                            e -= 1
                        step = 2.0 ** (e - 3)            # 3 mantissa bits
                        n = _py_round_even(a / step)      # exact: a/step is a scaled float
                        if e == -6 and a < 2.0 ** -6:
                            code = n                      # subnormal range, step 2^-9
                        else:
                            if n == 16:                   # carried into the next binade
                                e, n = e + 1, 8
                            code = ((e + 7) << 3) | (n - 8)
                        if math.copysign(1.0, y) < 0:
                            code |= 0x80
                        assert cache[b, h, dst[b] + t, d] == code, (b, t, h, d, y, code)
