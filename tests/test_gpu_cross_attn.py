"""GPU parity of wa_cross_attn (several decoder tokens attending to the
encoder frames, query and key lengths independent) against the oracle's
cross_attention, at the attention bar of tests/gpu_helpers.py (max-abs 2e-2
and mean-abs 2e-3 where M <= 1; 2^-7 M plus half a bf16 ulp on every
output)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attn
from tests.gpu_helpers import announce, assert_close, to_dev

pytestmark = pytest.mark.gpu


def _nan_out(B, T, H):
    return torch.full((B, T, H, 64), float("nan"), dtype=torch.bfloat16, device="cuda")


def _check(got, q, k, v, q_lens, k_lens, what, rows=None):
    """Compare the written rows with the oracle and check rows past q_lens
    are untouched (NaN).  rows: sequences to compare (None = all)."""
    B, Tq = q.shape[:2]
    Tk = k.shape[1]
    ql = np.clip(np.asarray(q_lens), 0, Tq)
    kl = np.clip(np.asarray(k_lens), 0, Tk)
    g = got.float().cpu().numpy()
    mask = np.arange(Tq)[None, :] < ql[:, None]
    assert np.all(np.isnan(g[~mask])), f"{what}: rows past q_lens were written"
    sel = np.arange(B) if rows is None else np.asarray(rows)
    want, mag = attn.cross_attention(q[sel].float().numpy(), k[sel].float().numpy(), v[sel].float().numpy(),
                                     ql[sel], kl[sel], 0.125, with_magnitude=True)
    m = mask[sel]
    if m.any():
        assert_close(torch.from_numpy(g[sel][m]), want[m], what, mag=mag[m])


def test_cross_ragged_lengths(gpu):
    """Query lengths across two 256-row query tiles, key lengths with ragged
    64-key tails, one key, no key (zero rows), no query, and lengths past
    the maxima or negative (clamped)."""
    import whisper_attention_amd as wa
    B, H, Tq, Tk = 8, 3, 300, 400
    q_lens = np.array([300, 1, 0, 257, 100, 64, 500, 33], np.int32)
    k_lens = np.array([400, 0, 5, 63, 129, 1, 999, -3], np.int32)
    announce(f"cross ragged B={B} H={H} Tq={Tq} Tk={Tk} q_lens={q_lens.tolist()} k_lens={k_lens.tolist()}")
    q, k, v = workloads.cross_inputs(B, H, Tq, Tk, 0.01, 20.0, seed=11)
    out = _nan_out(B, Tq, H)
    wa.wa_cross_attn(to_dev(q), to_dev(k), to_dev(v), out=out, q_lens=to_dev(q_lens), k_lens=to_dev(k_lens))
    torch.cuda.synchronize()
    _check(out, q, k, v, q_lens, k_lens, "cross ragged")
    g = out.float().cpu()
    assert torch.all(g[1, :1] == 0) and torch.all(g[7, :33] == 0), "rows with no key must be zero"


def test_cross_null_lengths_mean_full(gpu):
    import whisper_attention_amd as wa
    B, H, Tq, Tk = 2, 4, 70, 130
    announce(f"cross null lengths B={B} H={H} Tq={Tq} Tk={Tk}")
    q, k, v = workloads.cross_inputs(B, H, Tq, Tk, seed=12)
    out = _nan_out(B, Tq, H)
    wa.wa_cross_attn(to_dev(q), to_dev(k), to_dev(v), out=out)
    torch.cuda.synchronize()
    _check(out, q, k, v, [Tq] * B, [Tk] * B, "cross null lengths")


def test_cross_kv_in_cache_layout(gpu):
    """K and V as [B][H][Tk][64] caches, passed as transposed views; the
    output a view of wider storage."""
    import whisper_attention_amd as wa
    B, H, Tq, Tk = 3, 5, 40, 1500
    announce(f"cross K/V in cache layout B={B} H={H} Tq={Tq} Tk={Tk}")
    q, k, v = workloads.cross_inputs(B, H, Tq, Tk, 0.01, 20.0, seed=13)
    kc = to_dev(k.transpose(1, 2).contiguous())     # [B][H][Tk][64]
    vc = to_dev(v.transpose(1, 2).contiguous())
    big = torch.full((B, Tq, H + 3, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    view = big[:, :, 1:1 + H]
    q_lens = np.array([40, 17, 3], np.int32)
    k_lens = np.array([1500, 1000, 77], np.int32)
    wa.wa_cross_attn(to_dev(q), kc.transpose(1, 2), vc.transpose(1, 2), out=view, q_lens=to_dev(q_lens),
                     k_lens=to_dev(k_lens))
    torch.cuda.synchronize()
    _check(view, q, k, v, q_lens, k_lens, "cross cache layout")
    rest = torch.cat([big[:, :, :1], big[:, :, 1 + H:]], dim=2)
    assert torch.all(torch.isnan(rest.float())), "storage outside the view was written"


def test_cross_equal_lengths_is_encoder_attention(gpu):
    """With the same sequence for both lengths the call is the non-causal
    encoder attention: both go through one kernel, so the bits agree."""
    import whisper_attention_amd as wa
    B, H, T = 3, 2, 333
    lens = np.array([333, 200, 1], np.int32)
    announce(f"cross == encoder attention B={B} H={H} T={T}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=14)
    a, b = _nan_out(B, T, H), _nan_out(B, T, H)
    ld = to_dev(lens)
    wa.wa_cross_attn(to_dev(q), to_dev(k), to_dev(v), out=a, q_lens=ld, k_lens=ld)
    wa.wa_encoder_attn(to_dev(q), to_dev(k), to_dev(v), out=b, lens=ld, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_cross_prefill_full_size_sampled(gpu):
    """The prompt-prefill cross-attention: B=128 prompts of U[4,224] tokens,
    20 heads, against 1500 encoder frames, in the launch the benchmark times;
    eight sequences compared with the oracle."""
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["prefill_cross"]
    B, H, Tq, Tk = cfg["B"], cfg["H"], cfg["T"], cfg["T_k"]
    announce(f"cross prefill B={B} H={H} Tq={Tq} Tk={Tk}")
    q_lens = workloads.lens_uniform(B, cfg["lo"], cfg["hi"], 0)
    q, k, v = workloads.cross_inputs(B, H, Tq, Tk, cfg["outlier_p"], cfg["outlier_mult"], seed=0)
    out = _nan_out(B, Tq, H)
    wa.wa_cross_attn(to_dev(q), to_dev(k), to_dev(v), out=out, q_lens=to_dev(q_lens))
    torch.cuda.synchronize()
    rows = [0, 1, int(np.argmax(q_lens)), int(np.argmin(q_lens)), 50, 77, 100, 127]
    _check(out, q, k, v, q_lens, [Tk] * B, "cross prefill", rows=rows)


def test_cross_every_ring_position(gpu):
    """Key lengths of 1 to 14 tiles, whole and ragged, against query lengths
    that end at every 32-row wave of a 128-row tile."""
    import whisper_attention_amd as wa
    k_lens = np.array([64 * n + r for n in range(14) for r in (0, 17) if 64 * n + r > 0], np.int32)
    B, H, Tk = len(k_lens), 2, int(k_lens.max())
    q_lens = np.array([1 + (37 * i) % 160 for i in range(B)], np.int32)
    Tq = int(q_lens.max())
    announce(f"cross every ring position: B={B} Tq={Tq} Tk={Tk}")
    q, k, v = workloads.cross_inputs(B, H, Tq, Tk, seed=32)
    out = _nan_out(B, Tq, H)
    wa.wa_cross_attn(to_dev(q), to_dev(k), to_dev(v), out=out, q_lens=to_dev(q_lens), k_lens=to_dev(k_lens))
    torch.cuda.synchronize()
    _check(out, q, k, v, q_lens, k_lens, "cross ring positions")


def test_cross_over_a_dequantised_fp8_cache(gpu):
    """The composition the header describes for an fp8 cross cache: the
    encoder frames' K and V quantized into E4M3 caches (wa_kv_quant_fp8_kv,
    per-head dynamic scales), expanded back to bf16 (wa_kv_dequant_fp8), then
    the prompt's cross-attention over them (wa_cross_attn).  Codes, scales
    and the bf16 expansion bit for bit against the oracle's quantize and
    dequantise; the attention against the oracle's cross_attention over the
    oracle's expansion."""
    import whisper_attention_amd as wa
    from oracle import quant
    B, H, Tq, Tk = 4, 3, 40, 300
    announce(f"cross over a dequantised fp8 cache: B={B} H={H} Tq={Tq} Tk={Tk}")
    q, k, v = workloads.cross_inputs(B, H, Tq, Tk, 0.01, 20.0, seed=34)
    q_lens = np.array([40, 1, 17, 33], np.int32)
    full = np.full(B, Tk, np.int32)
    kc = torch.zeros((B, H, Tk, 64), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    ks = torch.zeros(H, dtype=torch.float32, device="cuda")
    vs = torch.zeros_like(ks)
    wa.wa_kv_quant_fp8_kv(to_dev(k), to_dev(v), kc, vc, ks, vs, "head", lens=to_dev(full))
    kd = torch.empty((B, Tk, H, 64), dtype=torch.bfloat16, device="cuda")
    vd = torch.empty_like(kd)
    wa.wa_kv_dequant_fp8(kc, ks, "head", "e4m3", out=kd, lens=to_dev(full))
    wa.wa_kv_dequant_fp8(vc, vs, "head", "e4m3", out=vd, lens=to_dev(full))
    out = _nan_out(B, Tq, H)
    wa.wa_cross_attn(to_dev(q), kd, vd, out=out, q_lens=to_dev(q_lens))
    torch.cuda.synchronize()
    ref = {}
    for name, x, c, s, d in (("K", k, kc, ks, kd), ("V", v, vc, vs, vd)):
        cache = np.zeros((B, H, Tk, 64), dtype=np.uint8)
        sc = quant.quantize_kv(x.float().numpy(), full, np.zeros(B, np.int64), cache, quant.PER_HEAD)
        assert np.array_equal(c.cpu().numpy(), cache), f"{name} codes"
        assert np.array_equal(s.cpu().numpy().view(np.uint32), sc.view(np.uint32)), f"{name} scales"
        bits = quant.unfill_cache(cache, full, sc, quant.PER_HEAD, Tk)
        assert np.array_equal(d.cpu().view(torch.int16).numpy().view(np.uint16), bits), f"{name} expansion"
        ref[name] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    _check(out, q, ref["K"], ref["V"], q_lens, full, "cross over dequantised fp8 cache")
