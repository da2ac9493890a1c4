"""GPU parity of wa_kv_quant_fp8 against the oracle: codes and scales bit-exact."""
import numpy as np
import pytest
import torch

import workloads
from oracle import quant
from tests.gpu_helpers import announce, to_dev

pytestmark = pytest.mark.gpu

GUARD = 0xA5


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    assert f.size == 65280
    return f


def _run_quant(wa, x_cpu, lens, dst, L, gran, scale_in=None, x_dev=None, fmt="e4m3"):
    """x_cpu: bf16 [B][T][H][64].  Returns (cache uint8 [B][H][L][64], scale float32)."""
    B, T, H, D = x_cpu.shape
    x = x_dev if x_dev is not None else to_dev(x_cpu)
    cache = torch.full((B, H, L, D), GUARD, dtype=torch.uint8, device="cuda")
    n = 1 if gran == "tensor" else H
    if scale_in is None:
        scale = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    else:
        scale = to_dev(np.asarray(scale_in, dtype=np.float32))
    lens_d = None if lens is None else to_dev(np.asarray(lens, dtype=np.int32))
    dst_d = None if dst is None else to_dev(np.asarray(dst, dtype=np.int32))
    if fmt == "e4m3":      # the E4M3 entry point itself
        wa.wa_kv_quant_fp8(x, cache, scale, gran, lens=lens_d, dst_start=dst_d,
                           compute_scale=scale_in is None)
    else:
        wa.wa_kv_quant_fp8_fmt(x, cache, scale, gran, fmt, lens=lens_d, dst_start=dst_d,
                               compute_scale=scale_in is None)
    torch.cuda.synchronize()
    return cache.cpu().numpy(), scale.cpu().numpy()


def _oracle(x_cpu, lens, dst, L, gran, scale_in=None, fmt="e4m3"):
    x = x_cpu.float().numpy()
    B, T, H, D = x.shape
    lens = np.full(B, T) if lens is None else np.asarray(lens)
    dst = np.zeros(B, dtype=np.int64) if dst is None else np.asarray(dst)
    g = quant.PER_TENSOR if gran == "tensor" else quant.PER_HEAD
    f = quant.E4M3 if fmt == "e4m3" else quant.E5M2
    cache = np.full((B, H, L, D), GUARD, dtype=np.uint8)
    if scale_in is None:
        s = quant.quantize_kv(x, lens, dst, cache, g, f)
    else:
        s = np.asarray(scale_in, dtype=np.float32)
        quant.fill_cache(x, lens, dst, cache, s, g, f)
    return cache, s


def _assert_same(got, want, what):
    gc, gs = got
    wc, ws = want
    assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32)), f"{what}: scales {gs} vs {ws}"
    bad = np.argwhere(gc != wc)
    assert bad.size == 0, f"{what}: {len(bad)} code mismatches, first at {bad[:4].tolist()}: " \
                          f"{gc[tuple(bad[0])]:#x} vs {wc[tuple(bad[0])]:#x}"


# 1/448 .. 93/448: the scales of N(0,1) data with and without x20 outliers;
# 2^-80 and 2^80 (and the float32 next to each, on the other side) bracket
# the range where the encoder takes the reciprocal path; 3e35 is the scale of
# the full bf16 range.
@pytest.mark.parametrize("s", [1.0, 0.125, 1.0 / 448, 4.25 / 448, 93.0 / 448, 2.0 ** -20 / 3,
                               2.0 ** -80, float(np.nextafter(np.float32(2.0 ** -80), np.float32(0))),
                               2.0 ** 80, float(np.nextafter(np.float32(2.0 ** 80), np.float32(np.inf))),
                               3.0e35])
def test_exhaustive_bf16_static_scale(gpu, s):
    import whisper_attention_amd as wa
    announce(f"quant exhaustive bf16, static scale {s}")
    x = torch.from_numpy(_all_finite_bf16().reshape(1, 1020, 1, 64)).to(torch.bfloat16)
    s32 = np.float32([s])
    _assert_same(_run_quant(wa, x, None, None, 1020, "tensor", s32),
                 _oracle(x, None, None, 1020, "tensor", s32), f"exhaustive s={s}")


def test_exhaustive_bf16_dynamic_scale(gpu):
    import whisper_attention_amd as wa
    announce("quant exhaustive bf16, dynamic scale")
    x = torch.from_numpy(_all_finite_bf16().reshape(1, 255, 4, 64)).to(torch.bfloat16)
    for gran in ("tensor", "head"):
        _assert_same(_run_quant(wa, x, None, None, 255, gran), _oracle(x, None, None, 255, gran),
                     f"exhaustive dynamic {gran}")
    # every bf16 of magnitude <= 16, whose dynamic scale 16/448 is an
    # ordinary one
    f = _all_finite_bf16()
    f = f[np.abs(f) <= 16.0]
    f = np.concatenate([f, np.zeros((-f.size) % 256, np.float32)])
    x = torch.from_numpy(f.reshape(1, -1, 4, 64)).to(torch.bfloat16)
    T = x.shape[1]
    for gran in ("tensor", "head"):
        _assert_same(_run_quant(wa, x, None, None, T, gran), _oracle(x, None, None, T, gran),
                     f"exhaustive |x|<=16 dynamic {gran}")


@pytest.mark.parametrize("which", ["self", "cross"])
def test_small_workload(gpu, which):
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["tiny"]
    T = cfg["self_len"] if which == "self" else cfg["T"]
    announce(f"quant small workload {which}: B=1 H=6 T={T} per-tensor")
    x = workloads.bf16_normal((1, T, cfg["H"], 64), 0, workloads.TID_KV_K)
    _assert_same(_run_quant(wa, x, [T], None, T, "tensor"), _oracle(x, [T], None, T, "tensor"),
                 f"small {which}")


@pytest.mark.parametrize("gran", ["head", "tensor"])
def test_prefill_fill_full_size(gpu, gran):
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["prefill"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    announce(f"quant prefill fill B={B} H={H} T={T} {gran}")
    lens = workloads.lens_uniform(B, cfg["lo"], cfg["hi"], 0)
    for tid in (workloads.TID_K, workloads.TID_V):
        x = workloads.bf16_normal((B, T, H, 64), 0, tid, cfg["outlier_p"], cfg["outlier_mult"])
        _assert_same(_run_quant(wa, x, lens, None, T, gran), _oracle(x, lens, None, T, gran),
                     f"prefill tid={tid} {gran}")


def test_ragged_dst_start_and_out_of_range_slots(gpu):
    import whisper_attention_amd as wa
    announce("quant ragged lens + dst_start + clipped slots")
    B, T, H, L = 5, 40, 4, 64
    x = workloads.bf16_normal((B, T, H, 64), 3, 77, 0.05, 20.0)
    lens = [40, 0, 1, 17, 40]
    dst = [0, 5, 63, 30, 50]          # seq 4 runs past slot 63: the tail is skipped
    for gran in ("tensor", "head"):
        _assert_same(_run_quant(wa, x, lens, dst, L, gran), _oracle(x, lens, dst, L, gran),
                     f"ragged {gran}")


def test_all_zero_input_gives_unit_scale(gpu):
    import whisper_attention_amd as wa
    announce("quant all-zero input")
    x = torch.zeros((2, 8, 3, 64), dtype=torch.bfloat16)
    x[1, 3, 2, 5] = -0.0
    for gran in ("tensor", "head"):
        got = _run_quant(wa, x, [8, 8], None, 8, gran)
        _assert_same(got, _oracle(x, [8, 8], None, 8, gran), f"zeros {gran}")
        assert np.all(got[1] == 1.0)


def test_strided_input_layout(gpu):
    import whisper_attention_amd as wa
    announce("quant strided [B][H][T][64] storage viewed as [B][T][H][64]")
    B, H, T = 3, 5, 33
    base = workloads.bf16_normal((B, H, T, 64), 4, 78)
    x_cpu = base.permute(0, 2, 1, 3)                      # [B][T][H][64] view
    x_dev = to_dev(base).permute(0, 2, 1, 3)
    lens = [33, 20, 7]
    got = _run_quant(wa, x_cpu, lens, None, T, "head", x_dev=x_dev)
    _assert_same(got, _oracle(x_cpu.contiguous(), lens, None, T, "head"), "strided")


def test_decode_append_with_static_scale(gpu):
    """One new token per sequence appended at slot lens-1 with the stored scales."""
    import whisper_attention_amd as wa
    announce("quant decode-step append, static per-head scale")
    B, H, L = 16, 20, 448
    lens = workloads.lens_uniform(B, 1, L, 5)
    x = workloads.bf16_normal((B, 1, H, 64), 5, 79, 0.01, 20.0)
    scale = workloads.scales_uniform(H, 5, 80)
    dst = lens - 1
    got = _run_quant(wa, x, np.ones(B, dtype=np.int32), dst, L, "head", scale_in=scale)
    _assert_same(got, _oracle(x, np.ones(B), dst, L, "head", scale_in=scale), "append")


def test_deterministic(gpu):
    import whisper_attention_amd as wa
    announce("quant determinism")
    x = workloads.bf16_normal((8, 100, 20, 64), 6, 81, 0.01, 20.0)
    a = _run_quant(wa, x, [100, 3, 50, 99, 1, 100, 64, 2], None, 100, "head")
    b = _run_quant(wa, x, [100, 3, 50, 99, 1, 100, 64, 2], None, 100, "head")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


@pytest.mark.parametrize("H", [1, 3, 17, 160])
def test_head_counts_and_block_shapes(gpu, H):
    """Row widths that give each block shape: lcm(64, 8H) threads (H=1, 3),
    8H rounded up to whole waves (H=17) and threads looping over pieces
    (H=160, rows wider than 1024 pieces)."""
    import whisper_attention_amd as wa
    B, T = 3, 37
    announce(f"quant head count H={H} B={B} T={T}")
    x = workloads.bf16_normal((B, T, H, 64), 9, 82, 0.02, 20.0)
    lens = [37, 1, 20]
    for gran in ("tensor", "head"):
        _assert_same(_run_quant(wa, x, lens, None, T, gran), _oracle(x, lens, None, T, gran),
                     f"H={H} {gran}")


def test_dynamic_scale_long_rows_one_head(gpu):
    """A dynamic scale over 139001 rows of one head: a large grid of amax
    blocks, so the last amax block folds thousands of partials per group."""
    import whisper_attention_amd as wa
    B, T, H = 2, 70000, 1
    announce(f"quant dynamic scale, B={B} T={T} H={H} (many partials)")
    x = workloads.bf16_normal((B, T, H, 64), 10, 83, 0.01, 20.0)
    lens = [70000, 69001]
    for gran in ("tensor", "head"):
        _assert_same(_run_quant(wa, x, lens, None, T, gran), _oracle(x, lens, None, T, gran),
                     f"long rows {gran}")


def _run_pair(wa, k_cpu, v_cpu, lens, dst, L, gran, fmt, scales_in=None, k_dev=None):
    B, T, H, D = k_cpu.shape
    kd = k_dev if k_dev is not None else to_dev(k_cpu)
    vd = to_dev(v_cpu)
    kc = torch.full((B, H, L, D), GUARD, dtype=torch.uint8, device="cuda")
    vc = torch.full_like(kc, GUARD)
    n = 1 if gran == "tensor" else H
    if scales_in is None:
        ks = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        vs = torch.full_like(ks, float("nan"))
    else:
        ks, vs = (to_dev(np.asarray(x, dtype=np.float32)) for x in scales_in)
    wa.wa_kv_quant_fp8_kv(kd, vd, kc, vc, ks, vs, gran, fmt,
                          lens=None if lens is None else to_dev(np.asarray(lens, dtype=np.int32)),
                          dst_start=None if dst is None else to_dev(np.asarray(dst, dtype=np.int32)),
                          compute_scale=scales_in is None)
    torch.cuda.synchronize()
    return (kc.cpu().numpy(), ks.cpu().numpy()), (vc.cpu().numpy(), vs.cpu().numpy())


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("gran", ["tensor", "head"])
def test_kv_pair_equals_two_fills(gpu, gran, fmt):
    """wa_kv_quant_fp8_kv: K (a strided view) and V (contiguous) in one call,
    each with its own scales, equal to two oracle fills; ragged lengths and
    slots, some clipped."""
    import whisper_attention_amd as wa
    announce(f"quant K/V pair {gran} {fmt}")
    B, T, H, L = 5, 40, 4, 64
    base = workloads.bf16_normal((B, H, T, 64), 7, 83, 0.05, 20.0)
    k_cpu = base.permute(0, 2, 1, 3)
    k_dev = to_dev(base).permute(0, 2, 1, 3)
    v_cpu = workloads.bf16_normal((B, T, H, 64), 7, 84, 0.0, 20.0) * 3
    lens, dst = [40, 0, 1, 17, 40], [0, 5, 63, 30, 50]
    got_k, got_v = _run_pair(wa, k_cpu, v_cpu, lens, dst, L, gran, fmt, k_dev=k_dev)
    _assert_same(got_k, _oracle(k_cpu.contiguous(), lens, dst, L, gran, fmt=fmt), f"pair K {gran} {fmt}")
    _assert_same(got_v, _oracle(v_cpu, lens, dst, L, gran, fmt=fmt), f"pair V {gran} {fmt}")


def test_kv_pair_prefill_full_size_and_static_scales(gpu):
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["prefill"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    announce(f"quant K/V pair prefill B={B} H={H} T={T} per head, then static scales")
    lens = workloads.lens_uniform(B, cfg["lo"], cfg["hi"], 0)
    k = workloads.bf16_normal((B, T, H, 64), 0, workloads.TID_K, cfg["outlier_p"], cfg["outlier_mult"])
    v = workloads.bf16_normal((B, T, H, 64), 0, workloads.TID_V, cfg["outlier_p"], cfg["outlier_mult"])
    got_k, got_v = _run_pair(wa, k, v, lens, None, T, "head", "e4m3")
    _assert_same(got_k, _oracle(k, lens, None, T, "head"), "pair prefill K")
    _assert_same(got_v, _oracle(v, lens, None, T, "head"), "pair prefill V")
    sk, sv = workloads.scales_uniform(H, 1, 85), workloads.scales_uniform(H, 1, 86)
    got_k, got_v = _run_pair(wa, k, v, lens, None, T, "head", "e4m3", scales_in=(sk, sv))
    _assert_same(got_k, _oracle(k, lens, None, T, "head", scale_in=sk), "pair static K")
    _assert_same(got_v, _oracle(v, lens, None, T, "head", scale_in=sv), "pair static V")
