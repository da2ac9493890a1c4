"""GPU parity of wa_encoder_attn_fp8qk (E4M3 Q and K, bf16 V) against the
oracle's attention over the dequantized codes, at the attention bar of
tests/gpu_helpers.py (max-abs 2e-2 and mean-abs 2e-3 where M <= 1; 2^-7 M
plus half a bf16 ulp on every output).  Codes and scales come from the oracle's quantize of
seeded bf16 Q and K (dynamic scales over the valid rows)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attn, quant
from tests.gpu_helpers import announce, assert_close, to_dev

pytestmark = pytest.mark.gpu

GRAN = {"tensor": quant.PER_TENSOR, "head": quant.PER_HEAD}


def _codes(x, lens, gran):
    xf = x.float().numpy()
    if lens is None:
        lens = np.full(xf.shape[0], xf.shape[1])
    s = quant.scales_from_amax(quant.group_amax(xf, lens, GRAN[gran]))
    return quant.quantize(xf, s, GRAN[gran]), s


def _run(wa, qc, qs, kc, ks, v, lens, causal, gran, views=None):
    B, T, H, D = v.shape
    if views is None:
        qd, kd, vd = to_dev(qc), to_dev(kc), to_dev(v)
    else:
        qd, kd, vd = views
    out = torch.full((B, T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    wa.wa_encoder_attn_fp8qk(qd, to_dev(qs), kd, to_dev(ks), gran, vd, out=out,
                             lens=None if lens is None else to_dev(np.asarray(lens, np.int32)),
                             causal=causal, softmax_scale=0.125)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _check(got, qc, qs, kc, ks, v, lens, causal, gran, what, pairs=None):
    B, T, H, _ = v.shape
    lens_a = np.full(B, T) if lens is None else np.asarray(lens)
    for b in range(B):
        assert np.all(np.isnan(got[b, lens_a[b]:])), f"{what}: rows past len written"
    g = GRAN[gran]
    if pairs is None:
        want, mag = attn.dense_attention_fp8qk(qc, qs, kc, ks, g, v.float().numpy(), lens_a, causal, 0.125,
                                               with_magnitude=True)
        mask = np.arange(T)[None, :] < lens_a[:, None]
        assert_close(torch.from_numpy(got[mask]), want[mask], what, mag=mag[mask])
        return
    gs, ws, ms = [], [], []
    for b, h in pairs:
        n = lens_a[b]
        sl = slice(h, h + 1)
        sq = qs[h:h + 1] if g == quant.PER_HEAD else qs
        sk = ks[h:h + 1] if g == quant.PER_HEAD else ks
        w, m = attn.dense_attention_fp8qk(qc[b:b + 1, :, sl], sq, kc[b:b + 1, :, sl], sk, g,
                                          v[b:b + 1, :, sl].float().numpy(), [n], causal, 0.125,
                                          with_magnitude=True)
        gs.append(got[b, :n, h])
        ws.append(w[0, :n, 0])
        ms.append(m[0, :n, 0])
    assert_close(torch.from_numpy(np.concatenate(gs)), np.concatenate(ws), what, mag=np.concatenate(ms))


def test_long_sequence(gpu):
    """4096 frames, 2 heads, per-head scales (two key groups of 32 tiles),
    all rows."""
    import whisper_attention_amd as wa
    lens = [4090]
    announce("fp8qk long sequence B=1 H=2 T=4096")
    q, k, v = workloads.encoder_inputs(1, 2, 4096, seed=38)
    qc, qs = _codes(q, lens, "head")
    kc, ks = _codes(k, lens, "head")
    got = _run(wa, qc, qs, kc, ks, v, lens, False, "head")
    _check(got, qc, qs, kc, ks, v, lens, False, "head", "fp8qk T=4096")


def test_two_key_groups_at_tile_edges(gpu):
    """Few blocks, so two key groups per block (merged in LDS), per-head
    scales; key lengths around the tile edges and the groups' split point."""
    import whisper_attention_amd as wa
    lens = [1, 64, 65, 128, 129, 192, 255, 256, 257, 300]
    B, H, T = len(lens), 2, 300
    announce(f"fp8qk two key groups B={B} H={H} T={T} lens={lens}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=34)
    qc, qs = _codes(q, lens, "head")
    kc, ks = _codes(k, lens, "head")
    got = _run(wa, qc, qs, kc, ks, v, lens, False, "head")
    _check(got, qc, qs, kc, ks, v, lens, False, "head", "fp8qk two key groups")


@pytest.mark.parametrize("gran", ["tensor", "head"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,T,lens", [(2, 3, 300, [300, 131]), (3, 2, 77, [77, 1, 64]), (1, 1, 1, [1]),
                                        (2, 2, 129, [0, 129]), (2, 1, 257, [257, 250])])
def test_ragged_shapes(gpu, B, H, T, lens, causal, gran):
    import whisper_attention_amd as wa
    announce(f"fp8qk ragged B={B} H={H} T={T} lens={lens} causal={causal} {gran}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=T + 1)
    qc, qs = _codes(q, lens, gran)
    kc, ks = _codes(k, lens, gran)
    got = _run(wa, qc, qs, kc, ks, v, lens, causal, gran)
    _check(got, qc, qs, kc, ks, v, lens, causal, gran, f"fp8qk B={B} T={T} causal={causal} {gran}")


def test_large_v3_encoder_full_size(gpu):
    """Every (b, h) of the 30-s shape, element by element."""
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["enc_l3"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    announce(f"fp8qk encoder large-v3 B={B} H={H} T={T} per-tensor (every (b, h))")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=0)
    qc, qs = _codes(q, None, "tensor")
    kc, ks = _codes(k, None, "tensor")
    got = _run(wa, qc, qs, kc, ks, v, None, False, "tensor")
    assert np.all(np.isfinite(got))
    pairs = [(b, h) for b in range(B) for h in range(H)]
    _check(got, qc, qs, kc, ks, v, None, False, "tensor", "fp8qk enc-L3", pairs=pairs)


def test_prefill_causal_full_size_per_head(gpu):
    """The prefill shape (B=128 H=20 T=224, lengths U[4,224]) with x20
    outliers in K, per-head scales, causal."""
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["prefill"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    announce(f"fp8qk prefill B={B} H={H} T={T} causal per-head")
    lens = workloads.lens_uniform(B, cfg["lo"], cfg["hi"], 0)
    q, k, v = workloads.prefill_inputs(B, H, T, cfg["lo"], cfg["hi"], cfg["outlier_p"], cfg["outlier_mult"],
                                       seed=0)[:3]
    qc, qs = _codes(q, lens, "head")
    kc, ks = _codes(k, lens, "head")
    got = _run(wa, qc, qs, kc, ks, v, lens, True, "head")
    _check(got, qc, qs, kc, ks, v, lens, True, "head", "fp8qk prefill")


def test_codes_from_the_quantize_kernel_and_strided_views(gpu):
    """Q and K codes written by wa_kv_quant_fp8 into [B][T][H][64] storage
    (cache strides over that layout), then read by the attention through
    views of wider storage.  The kernel's codes and scales must equal the
    oracle's bit for bit; the expected output uses the oracle's."""
    import whisper_attention_amd as wa
    B, H, T = 3, 4, 200
    announce(f"fp8qk codes from the quantize kernel B={B} H={H} T={T}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=21)
    lens = [200, 150, 33]
    ld = to_dev(np.asarray(lens, np.int32))
    big = torch.zeros((2, B, T, H + 2, 64), dtype=torch.uint8, device="cuda")
    qv, kv = big[0, :, :, 1:H + 1], big[1, :, :, 1:H + 1]          # [B][T][H][64] views
    qsd = torch.zeros(H, dtype=torch.float32, device="cuda")
    ksd = torch.zeros(H, dtype=torch.float32, device="cuda")
    wa.wa_kv_quant_fp8(to_dev(q), qv.permute(0, 2, 1, 3), qsd, "head", lens=ld)
    wa.wa_kv_quant_fp8(to_dev(k), kv.permute(0, 2, 1, 3), ksd, "head", lens=ld)
    vd = to_dev(v)
    out = torch.full((B, T, H, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    wa.wa_encoder_attn_fp8qk(qv, qsd, kv, ksd, "head", vd, out=out, lens=ld, causal=False, softmax_scale=0.125)
    torch.cuda.synchronize()
    qc, qs = _codes(q, lens, "head")
    kc, ks = _codes(k, lens, "head")
    valid = np.arange(T)[None, :] < np.asarray(lens)[:, None]
    for got_c, want_c, got_s, want_s in ((qv, qc, qsd, qs), (kv, kc, ksd, ks)):
        assert np.array_equal(got_s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
        assert np.array_equal(got_c.cpu().numpy()[valid], want_c[valid])
    _check(out.float().cpu().numpy(), qc, qs, kc, ks, v, lens, False, "head", "fp8qk from quantize kernel")


@pytest.mark.parametrize("causal", [False, True])
def test_every_ring_position(gpu, causal):
    """fp8 K tiles through every position of the unrolled tile loop (1 to 14
    tiles, whole and ragged), per-head scales."""
    import whisper_attention_amd as wa
    lens = [64 * n + r for n in range(14) for r in (0, 17) if 64 * n + r > 0]
    B, H, T = len(lens), 2, max(lens)
    announce(f"fp8qk every ring position, causal={causal}: B={B} T={T}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=33)
    qc, qs = _codes(q, lens, "head")
    kc, ks = _codes(k, lens, "head")
    got = _run(wa, qc, qs, kc, ks, v, lens, causal, "head")
    _check(got, qc, qs, kc, ks, v, lens, causal, "head", f"fp8qk ring positions causal={causal}")
