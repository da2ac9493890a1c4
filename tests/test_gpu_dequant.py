"""GPU parity of the E5M2 quantize (wa_kv_quant_fp8_fmt) and of the dequantise
(wa_kv_dequant_fp8, both formats) against the oracle, bit for bit.

NaN codes (never written by the quantize calls) are compared as NaN-ness only.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import quant
from tests.gpu_helpers import announce, to_dev
from tests.test_gpu_quant import _all_finite_bf16, _assert_same, _oracle, _run_quant

pytestmark = pytest.mark.gpu

SENTINEL = 0xFFFF
FMTS = ["e4m3", "e5m2"]
OFMT = {"e4m3": quant.E4M3, "e5m2": quant.E5M2}


# ---- E5M2 quantize -----------------------------------------------------------

# 1/57344 .. 93/57344: the scales of N(0,1) data with and without x20
# outliers; 2^-80 and 2^80 (and the float32 next to each, on the other side)
# bracket the reciprocal path; 6e33 is the scale of the full bf16 range.
@pytest.mark.parametrize("s", [1.0, 0.125, 1.0 / 57344, 4.25 / 57344, 93.0 / 57344, 2.0 ** -20 / 3,
                               2.0 ** -80, float(np.nextafter(np.float32(2.0 ** -80), np.float32(0))),
                               2.0 ** 80, float(np.nextafter(np.float32(2.0 ** 80), np.float32(np.inf))),
                               6.0e33])
def test_e5m2_exhaustive_bf16_static_scale(gpu, s):
    import whisper_attention_amd as wa
    announce(f"e5m2 quant exhaustive bf16, static scale {s}")
    x = torch.from_numpy(_all_finite_bf16().reshape(1, 1020, 1, 64)).to(torch.bfloat16)
    s32 = np.float32([s])
    _assert_same(_run_quant(wa, x, None, None, 1020, "tensor", s32, fmt="e5m2"),
                 _oracle(x, None, None, 1020, "tensor", s32, fmt="e5m2"), f"e5m2 exhaustive s={s}")


def test_e5m2_exhaustive_bf16_dynamic_scale(gpu):
    import whisper_attention_amd as wa
    announce("e5m2 quant exhaustive bf16, dynamic scale")
    x = torch.from_numpy(_all_finite_bf16().reshape(1, 255, 4, 64)).to(torch.bfloat16)
    for gran in ("tensor", "head"):
        _assert_same(_run_quant(wa, x, None, None, 255, gran, fmt="e5m2"),
                     _oracle(x, None, None, 255, gran, fmt="e5m2"), f"e5m2 exhaustive dynamic {gran}")
    f = _all_finite_bf16()
    f = f[np.abs(f) <= 16.0]
    f = np.concatenate([f, np.zeros((-f.size) % 256, np.float32)])
    x = torch.from_numpy(f.reshape(1, -1, 4, 64)).to(torch.bfloat16)
    T = x.shape[1]
    for gran in ("tensor", "head"):
        _assert_same(_run_quant(wa, x, None, None, T, gran, fmt="e5m2"),
                     _oracle(x, None, None, T, gran, fmt="e5m2"), f"e5m2 |x|<=16 dynamic {gran}")


@pytest.mark.parametrize("gran", ["head", "tensor"])
def test_e5m2_prefill_fill_full_size(gpu, gran):
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["prefill"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    announce(f"e5m2 quant prefill fill B={B} H={H} T={T} {gran}")
    lens = workloads.lens_uniform(B, cfg["lo"], cfg["hi"], 0)
    x = workloads.bf16_normal((B, T, H, 64), 0, workloads.TID_K, cfg["outlier_p"], cfg["outlier_mult"])
    _assert_same(_run_quant(wa, x, lens, None, T, gran, fmt="e5m2"),
                 _oracle(x, lens, None, T, gran, fmt="e5m2"), f"e5m2 prefill {gran}")


def test_e5m2_ragged_dst_start(gpu):
    import whisper_attention_amd as wa
    announce("e5m2 quant ragged lens + dst_start + clipped slots")
    B, T, H, L = 5, 40, 4, 64
    x = workloads.bf16_normal((B, T, H, 64), 3, 77, 0.05, 20.0)
    lens, dst = [40, 0, 1, 17, 40], [0, 5, 63, 30, 50]
    for gran in ("tensor", "head"):
        _assert_same(_run_quant(wa, x, lens, dst, L, gran, fmt="e5m2"),
                     _oracle(x, lens, dst, L, gran, fmt="e5m2"), f"e5m2 ragged {gran}")


# ---- dequantise --------------------------------------------------------------

def _run_dequant(wa, cache_np, scale_np, gran, fmt, T, lens=None, out=None):
    cache = to_dev(cache_np)
    scale = to_dev(np.asarray(scale_np, dtype=np.float32))
    B, H, L, D = cache_np.shape
    if out is None:
        out = torch.full((B, T, H, D), SENTINEL, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
        out = out.to("cuda")
    lens_d = None if lens is None else to_dev(np.asarray(lens, dtype=np.int32))
    wa.wa_kv_dequant_fp8(cache, scale, gran, fmt, out=out, lens=lens_d)
    torch.cuda.synchronize()
    return out


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _want(cache_np, scale_np, gran, fmt, T, lens):
    B = cache_np.shape[0]
    lens = np.full(B, T) if lens is None else np.asarray(lens)
    g = quant.PER_TENSOR if gran == "tensor" else quant.PER_HEAD
    return quant.unfill_cache(cache_np, lens, np.asarray(scale_np, np.float32), g, T, OFMT[fmt])


def _assert_bits(got, want, what):
    gv = (got.astype(np.uint32) << 16).view(np.float32)
    wv = (want.astype(np.uint32) << 16).view(np.float32)
    nan = np.isnan(gv) & np.isnan(wv)
    bad = np.argwhere((got != want) & ~nan)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:4].tolist()}: " \
                          f"{got[tuple(bad[0])]:#06x} vs {want[tuple(bad[0])]:#06x}"


def _every_code_cache(B, H, L, seed):
    """[B][H][L][64] holding every code many times, in a shuffled order."""
    n = B * H * L * 64
    codes = np.tile(np.arange(256, dtype=np.uint8), -(-n // 256))[:n]
    workloads.rng(seed, 90).shuffle(codes)
    return codes.reshape(B, H, L, 64)


# products in the fp32 subnormal range, near the fp32 top, and ordinary ones
DQ_SCALES = [1.0, 0.125, 1.0 / 448, 93.0 / 57344, 3.0e-3, float.fromhex("0x1.8p-120"),
             float.fromhex("0x1.fffffep100")]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("s", DQ_SCALES)
def test_dequant_every_code_per_tensor(gpu, fmt, s):
    import whisper_attention_amd as wa
    announce(f"dequant every code {fmt} scale {s}")
    cache = _every_code_cache(2, 3, 70, 1)
    got = _bits(_run_dequant(wa, cache, [s], "tensor", fmt, 70))
    _assert_bits(got, _want(cache, [s], "tensor", fmt, 70, None), f"{fmt} s={s}")


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_every_code_per_head(gpu, fmt):
    import whisper_attention_amd as wa
    announce(f"dequant every code {fmt} per-head scales")
    H = len(DQ_SCALES)
    cache = _every_code_cache(2, H, 40, 2)
    got = _bits(_run_dequant(wa, cache, DQ_SCALES, "head", fmt, 40))
    _assert_bits(got, _want(cache, DQ_SCALES, "head", fmt, 40, None), f"{fmt} per head")


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_ragged_lengths_and_bounds(gpu, fmt):
    """lens below, at and past the cache length (clamped), negative and zero;
    T_max below and above cache_len; positions at or past n keep the sentinel."""
    import whisper_attention_amd as wa
    B, H, L = 6, 5, 300
    cache = _every_code_cache(B, H, L, 3)
    lens = [0, 1, 129, 300, 1000, -4]
    scale = workloads.scales_uniform(H, 3, 91)
    for T in (300, 200, 333):
        announce(f"dequant ragged {fmt} T_max={T} cache_len={L}")
        got = _bits(_run_dequant(wa, cache, scale, "head", fmt, T, lens))
        want = _want(cache, scale, "head", fmt, T, lens)
        _assert_bits(got, want, f"{fmt} ragged T={T}")
        assert np.all(got[:, min(T, L):] == SENTINEL)


def test_dequant_strided_output(gpu):
    """The output is a [B][T][H][64] view of wider storage (heads 2..6 of 9)."""
    import whisper_attention_amd as wa
    announce("dequant into a strided view")
    B, H, L = 3, 5, 77
    cache = _every_code_cache(B, H, L, 4)
    big = torch.full((B, L, 9, 64), SENTINEL, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    big = big.to("cuda")
    view = big[:, :, 2:7, :]
    scale = [0.01]
    _run_dequant(wa, cache, scale, "tensor", "e4m3", L, lens=[77, 10, 0], out=view)
    got = _bits(big)
    want = _want(cache, scale, "tensor", "e4m3", L, [77, 10, 0])
    _assert_bits(got[:, :, 2:7], want, "strided view")
    assert np.all(got[:, :, :2] == SENTINEL) and np.all(got[:, :, 7:] == SENTINEL)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_prefill_cache_full_size(gpu, fmt):
    """The prefill cache (B=128 H=20 T=224, lengths U[4,224], per-head),
    filled on the CPU by the oracle's quantize of bf16 data with outliers."""
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["prefill"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    announce(f"dequant prefill cache {fmt} B={B} H={H} T={T}")
    lens = workloads.lens_uniform(B, cfg["lo"], cfg["hi"], 0)
    x = workloads.bf16_normal((B, T, H, 64), 0, workloads.TID_V, cfg["outlier_p"], cfg["outlier_mult"])
    cache = np.zeros((B, H, T, 64), dtype=np.uint8)
    scale = quant.quantize_kv(x.float().numpy(), lens, np.zeros(B, np.int64), cache, quant.PER_HEAD,
                              OFMT[fmt])
    got = _bits(_run_dequant(wa, cache, scale, "head", fmt, T, lens))
    _assert_bits(got, _want(cache, scale, "head", fmt, T, lens), f"prefill {fmt}")


def test_dequant_cross_cache_full_size_sampled(gpu):
    """The decode cross cache (B=64 H=20 L=1500, E4M3 codes shaped like a
    quantized bell curve): the whole cache is read back, four sequences are
    compared with the oracle and every position is written."""
    import whisper_attention_amd as wa
    B, H, L = 64, 20, 1500
    announce(f"dequant cross cache B={B} H={H} L={L}")
    cache = workloads.fp8_codes((B, H, L, 64), 0, workloads.TID_XK_CODES).numpy()
    scale = workloads.scales_uniform(1, 0, workloads.TID_XK_SCALE)
    got = _bits(_run_dequant(wa, cache, scale, "tensor", "e4m3", L))
    assert not np.any(got == SENTINEL)
    for b in (0, 17, 42, 63):
        want = _want(cache[b:b + 1], scale, "tensor", "e4m3", L, None)
        _assert_bits(got[b:b + 1], want, f"cross b={b}")
