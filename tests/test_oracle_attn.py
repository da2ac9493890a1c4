"""Pins for the oracle's attention functions.

Against: pure-Python fp64 loops on tiny shapes (causal, non-causal, ragged,
empty); the softmax invariants (equal scores -> mean of V, one dominant key
-> its V row, a constant added to every score changes nothing, one key -> its
V row, key permutation, linearity in V); torch's scaled_dot_product_attention
in float64 at the small workload's size; the decode query as the last row of
causal attention; the split-key merge identity.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attn, quant
import workloads


def _brute_dense(q, k, v, lens, causal, sc):
    B, T, H, D = q.shape
    out = np.full(q.shape, np.nan)
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            for i in range(n):
                keys = range(i + 1) if causal else range(n)
                s = [sc * sum(float(q[b, i, h, d]) * float(k[b, j, h, d]) for d in range(D)) for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = sum(w)
                for d in range(D):
                    out[b, i, h, d] = sum(w[t] * float(v[b, j, h, d]) for t, j in enumerate(keys)) / z
    return out


@pytest.mark.parametrize("D", [1, 4, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_vs_brute_force(D, causal):
    g = np.random.default_rng(D + 10 * causal)
    B, T, H = 3, 9, 2
    q, k, v = (g.standard_normal((B, T, H, D)) for _ in range(3))
    lens = np.array([9, 5, 1])
    sc = 1.0 / math.sqrt(D)
    got = attn.dense_attention(q, k, v, lens, causal, sc)
    want = _brute_dense(q, k, v, lens, causal, sc)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    np.testing.assert_allclose(got[fin], want[fin], rtol=1e-12, atol=1e-12)


def test_dense_empty_sequence_has_no_rows():
    q = np.ones((2, 4, 1, 64))
    out = attn.dense_attention(q, q, q, np.array([0, 4]), False, 0.125)
    assert np.all(np.isnan(out[0])) and not np.any(np.isnan(out[1]))


def test_equal_scores_give_mean_of_v():
    g = np.random.default_rng(1)
    T = 33
    q = g.standard_normal((1, T, 1, 64))
    krow = g.standard_normal(64)
    k = np.broadcast_to(krow, (1, T, 1, 64)).copy()
    v = g.standard_normal((1, T, 1, 64))
    out = attn.dense_attention(q, k, v, [T], False, 0.125)
    np.testing.assert_allclose(out[0, :, 0], np.broadcast_to(v[0, :, 0].mean(0), (T, 64)), atol=1e-12)
    out_c = attn.dense_attention(q, k, v, [T], True, 0.125)
    for i in range(T):
        np.testing.assert_allclose(out_c[0, i, 0], v[0, :i + 1, 0].mean(0), atol=1e-12)


def test_dominant_key_gives_its_v_row():
    g = np.random.default_rng(2)
    T, j0 = 20, 7
    q = np.zeros((1, T, 1, 64))
    q[..., 0] = 1.0
    k = g.standard_normal((1, T, 1, 64)) * 0.1
    k[0, j0, 0, 0] = 8.0 * 60           # score margin >= 50 after the 1/8 scale
    v = g.standard_normal((1, T, 1, 64))
    out = attn.dense_attention(q, k, v, [T], False, 0.125)
    np.testing.assert_allclose(out[0, :, 0], np.broadcast_to(v[0, j0, 0], (T, 64)), atol=1e-15)


def test_constant_shift_of_scores_is_invisible():
    g = np.random.default_rng(3)
    L = 40
    q = g.standard_normal((1, 1, 64))
    kh = g.standard_normal((1, 1, L, 64))
    vh = g.standard_normal((1, 1, L, 64))
    c = 3.7
    # adding c * q / |q|^2 to every key adds c * softmax_scale to every score
    kh2 = kh + c * q[0, 0] / (q[0, 0] @ q[0, 0])
    a = attn.decode_attention_dequant(q, kh, vh, [L], 0.125)
    b = attn.decode_attention_dequant(q, kh2, vh, [L], 0.125)
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_single_key_and_permutation_and_linearity():
    g = np.random.default_rng(4)
    T = 17
    q, k, v, v2 = (g.standard_normal((1, T, 2, 64)) for _ in range(4))
    one = attn.dense_attention(q[:, :1], k[:, :1], v[:, :1], [1], False, 0.125)
    np.testing.assert_allclose(one[0, 0], v[0, 0], atol=1e-15)
    perm = g.permutation(T)
    a = attn.dense_attention(q, k, v, [T], False, 0.125)
    b = attn.dense_attention(q, k[:, perm], v[:, perm], [T], False, 0.125)
    np.testing.assert_allclose(a, b, atol=1e-12)
    c = attn.dense_attention(q, k, 2.0 * v - 3.0 * v2, [T], False, 0.125)
    d = 2.0 * a - 3.0 * attn.dense_attention(q, k, v2, [T], False, 0.125)
    np.testing.assert_allclose(c, d, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_dense_vs_torch_sdpa_float64_small_workload(causal):
    cfg = workloads.CONFIGS["tiny"]
    q, k, v = workloads.encoder_inputs(cfg["B"], cfg["H"], cfg["T"], seed=0)
    qf, kf, vf = (t.float().numpy() for t in (q, k, v))
    T = cfg["T"]
    got = attn.dense_attention(qf, kf, vf, [T], causal, 0.125)
    tq, tk, tv = (t.double().permute(0, 2, 1, 3) for t in (q, k, v))     # [B][H][T][D]
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.125)
    want = want.permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_decode_is_last_row_of_causal_attention():
    g = np.random.default_rng(5)
    B, H, L = 3, 2, 12
    lens = np.array([12, 5, 1])
    kc = workloads.fp8_codes((B, H, L, 64), 0, 99).numpy()
    vc = workloads.fp8_codes((B, H, L, 64), 0, 98).numpy()
    ks = np.float32([0.01, 0.02])
    vs = np.float32([0.03, 0.005])
    q = g.standard_normal((B, H, 64)).astype(np.float32)
    got = attn.decode_attention(q, kc, vc, ks, vs, quant.PER_HEAD, lens, 0.125)
    khat = quant.dequantize(kc, ks, quant.PER_HEAD, head_axis=1)
    vhat = quant.dequantize(vc, vs, quant.PER_HEAD, head_axis=1)
    for b in range(B):
        n = lens[b]
        Q = np.zeros((1, n, H, 64))
        Q[0, n - 1] = q[b]
        K = khat[b, :, :n].transpose(1, 0, 2)[None]
        V = vhat[b, :, :n].transpose(1, 0, 2)[None]
        want = attn.dense_attention(Q, K, V, [n], True, 0.125)[0, n - 1]
        np.testing.assert_allclose(got[b], want, rtol=1e-12, atol=1e-12)
    # one cached token: the output is that token's dequantized V row
    one = attn.decode_attention(q, kc, vc, ks, vs, quant.PER_HEAD, np.array([1, 1, 1]), 0.125)
    np.testing.assert_allclose(one, vhat[:, :, 0], atol=1e-15)
    # zero cached tokens: a zero row
    zero = attn.decode_attention(q, kc, vc, ks, vs, quant.PER_HEAD, np.array([0, 3, 0]), 0.125)
    assert np.all(zero[0] == 0) and np.all(zero[2] == 0)


def test_decode_dequant_is_code_times_scale():
    # per-tensor: the scale multiplies every decoded code, checked on a brute
    # force dot product for one (b, h)
    kc = workloads.fp8_codes((1, 1, 3, 64), 0, 97).numpy()
    vc = workloads.fp8_codes((1, 1, 3, 64), 0, 96).numpy()
    q = np.linspace(-1, 1, 64).reshape(1, 1, 64)
    ks, vs = np.float32([0.0125]), np.float32([0.25])
    from oracle import e4m3
    got = attn.decode_attention(q, kc, vc, ks, vs, quant.PER_TENSOR, [3], 0.125)
    s = [0.125 * sum(q[0, 0, d] * e4m3.decode(kc[0, 0, j, d]) * float(ks[0]) for d in range(64)) for j in range(3)]
    w = [math.exp(x - max(s)) for x in s]
    want = [sum(w[j] * e4m3.decode(vc[0, 0, j, d]) * float(vs[0]) for j in range(3)) / sum(w) for d in range(64)]
    np.testing.assert_allclose(got[0, 0], want, rtol=1e-12)


@pytest.mark.parametrize("cuts", [[0, 1500], [0, 256, 512, 768, 1024, 1280, 1500], [0, 1, 2, 999, 1500]])
def test_split_key_merge_identity(cuts):
    g = np.random.default_rng(6)
    L = 1500
    q = g.standard_normal(64)
    kh = g.standard_normal((L, 64)) * 0.5
    vh = g.standard_normal((L, 64))
    parts = [attn.decode_partial(q, kh[a:b], vh[a:b], 0.125) for a, b in zip(cuts[:-1], cuts[1:])]
    merged = attn.merge_partials(*zip(*parts))
    full = attn.decode_attention_dequant(q.reshape(1, 1, 64), kh.reshape(1, 1, L, 64),
                                         vh.reshape(1, 1, L, 64), [L], 0.125)[0, 0]
    np.testing.assert_allclose(merged, full, rtol=1e-12, atol=1e-14)


def test_magnitude_is_weighted_abs_v():
    """The tolerance normaliser: equals O when V >= 0, bounds |O|, and matches
    a brute-force weighted mean of |V|."""
    g = np.random.default_rng(7)
    q, k, v = (g.standard_normal((2, 9, 2, 4)) for _ in range(3))
    lens = np.array([9, 4])
    out, mag = attn.dense_attention(q, k, v, lens, True, 0.5, with_magnitude=True)
    out_abs, mag_abs = attn.dense_attention(q, k, np.abs(v), lens, True, 0.5, with_magnitude=True)
    fin = ~np.isnan(out)
    np.testing.assert_allclose(mag_abs[fin], out_abs[fin], rtol=1e-13)
    np.testing.assert_allclose(mag[fin], mag_abs[fin], rtol=1e-13)
    assert np.all(mag[fin] >= np.abs(out[fin]) - 1e-13)
    want = _brute_dense(q, k, np.abs(v), lens, True, 0.5)
    np.testing.assert_allclose(mag[fin], want[fin], rtol=1e-12)
    qd = g.standard_normal((2, 2, 4))
    kh, vh = g.standard_normal((2, 2, 5, 4)), g.standard_normal((2, 2, 5, 4))
    o2, m2 = attn.decode_attention_dequant(qd, kh, vh, [5, 2], 0.5, with_magnitude=True)
    o3 = attn.decode_attention_dequant(qd, kh, np.abs(vh), [5, 2], 0.5)
    np.testing.assert_allclose(m2, o3, rtol=1e-13)


@pytest.mark.parametrize("gran", [quant.PER_TENSOR, quant.PER_HEAD])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8qk_is_attention_on_code_times_scale(gran, causal):
    """Brute force with Python scalars on a tiny ragged batch: scores from
    the decoded E4M3 codes times their scales (the per-head scale of head h
    for both operands), the softmax, V in full precision."""
    from oracle import e4m3
    B, T, H, D = 2, 5, 2, 4
    qc = workloads.fp8_codes((B, T, H, D), 3, 91).numpy()
    kc = workloads.fp8_codes((B, T, H, D), 3, 92).numpy()
    v = np.random.default_rng(5).standard_normal((B, T, H, D))
    qs = np.float32([0.02, 0.5])[: (1 if gran == quant.PER_TENSOR else 2)]
    ks = np.float32([0.25, 0.003])[: (1 if gran == quant.PER_TENSOR else 2)]
    lens = [5, 3]
    got = attn.dense_attention_fp8qk(qc, qs, kc, ks, gran, v, lens, causal, 0.125)
    for b in range(B):
        for h in range(H):
            g = 0 if gran == quant.PER_TENSOR else h
            for i in range(lens[b]):
                keys = range(i + 1) if causal else range(lens[b])
                s = [0.125 * sum(e4m3.decode(qc[b, i, h, d]) * float(qs[g]) *
                                 e4m3.decode(kc[b, j, h, d]) * float(ks[g]) for d in range(D)) for j in keys]
                w = [math.exp(x - max(s)) for x in s]
                want = [sum(w[t] * v[b, j, h, d] for t, j in enumerate(keys)) / sum(w) for d in range(D)]
                np.testing.assert_allclose(got[b, i, h], want, rtol=1e-12, atol=1e-14)


def test_fp8qk_scale_moves_between_q_and_k_and_softmax_scale():
    """Only the product softmax_scale * q_scale * k_scale matters."""
    B, T, H, D = 1, 7, 1, 64
    qc = workloads.fp8_codes((B, T, H, D), 4, 93).numpy()
    kc = workloads.fp8_codes((B, T, H, D), 4, 94).numpy()
    v = np.random.default_rng(6).standard_normal((B, T, H, D))
    a = attn.dense_attention_fp8qk(qc, np.float32([0.01]), kc, np.float32([0.04]), quant.PER_TENSOR, v,
                                   [7], False, 0.125)
    b = attn.dense_attention_fp8qk(qc, np.float32([0.04]), kc, np.float32([0.02]), quant.PER_TENSOR, v,
                                   [7], False, 0.0625)
    np.testing.assert_allclose(a, b, rtol=1e-12)


def test_cross_attention_brute_force_ragged():
    """Pure-Python loops: query rows below q_lens attend to keys below k_lens."""
    g = np.random.default_rng(31)
    B, Tq, Tk, H, D = 3, 5, 9, 2, 4
    q = g.standard_normal((B, Tq, H, D))
    k = g.standard_normal((B, Tk, H, D))
    v = g.standard_normal((B, Tk, H, D))
    ql, kl = [5, 2, 0], [9, 1, 4]
    got = attn.cross_attention(q, k, v, ql, kl, 0.3)
    for b in range(B):
        assert np.all(np.isnan(got[b, ql[b]:]))
        for h in range(H):
            for i in range(ql[b]):
                s = [0.3 * sum(q[b, i, h, d] * k[b, j, h, d] for d in range(D)) for j in range(kl[b])]
                w = [math.exp(x - max(s)) for x in s]
                want = [sum(w[j] * v[b, j, h, d] for j in range(kl[b])) / sum(w) for d in range(D)]
                np.testing.assert_allclose(got[b, i, h], want, rtol=1e-12, atol=1e-14)


def test_cross_attention_special_cases():
    g = np.random.default_rng(32)
    B, T, H, D = 2, 11, 3, 64
    q, k, v = (g.standard_normal((B, T, H, D)) for _ in range(3))
    lens = np.array([11, 6])
    # equal query and key lengths: the non-causal dense attention
    np.testing.assert_allclose(attn.cross_attention(q, k, v, lens, lens, 0.125),
                               attn.dense_attention(q, k, v, lens, False, 0.125), rtol=1e-12, equal_nan=True)
    # no keys: zero rows
    z = attn.cross_attention(q, k, v, [3, 0], [0, 5], 0.125)
    assert np.all(z[0, :3] == 0) and np.all(np.isnan(z[0, 3:])) and np.all(np.isnan(z[1]))
    # one query row: the decode attention over the same (unquantized) keys
    one = attn.cross_attention(q[:, :1], k, v, [1, 1], lens, 0.125)
    dec = attn.decode_attention_dequant(q[:, 0], np.transpose(k, (0, 2, 1, 3)), np.transpose(v, (0, 2, 1, 3)),
                                        lens, 0.125)
    np.testing.assert_allclose(one[:, 0], dec, rtol=1e-12)
