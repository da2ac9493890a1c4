"""GPU parity on seeded random shapes: sizes, lengths, masks, scale groups
and variants drawn per case, each compared with the oracle at the usual bar
(attention: max-abs 2e-2 and mean-abs 2e-3 where M <= 1, and 2^-7 M plus
half a bf16 ulp on every output, as tests/gpu_helpers.py states; codes: bit
for bit).  The shapes stay small enough for the oracle to finish in seconds
while still spanning several tiles and ragged tails."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attn, quant
from tests.gpu_helpers import announce, assert_close, to_dev

pytestmark = pytest.mark.gpu

GRAN = {"tensor": quant.PER_TENSOR, "head": quant.PER_HEAD}


def _case_rng(kind, i):
    return np.random.default_rng([2024, kind, i])


@pytest.mark.parametrize("i", range(10))
def test_encoder_random(gpu, i):
    import whisper_attention_amd as wa
    g = _case_rng(1, i)
    B, H = int(g.integers(1, 4)), int(g.integers(1, 5))
    T = int(g.integers(1, 700))
    lens = g.integers(0, T + 1, size=B).astype(np.int32)
    lens[g.integers(B)] = T
    causal = bool(g.integers(2))
    fp8 = bool(g.integers(2))
    gran = ["tensor", "head"][int(g.integers(2))]
    announce(f"random encoder #{i}: B={B} H={H} T={T} lens={lens.tolist()} causal={causal} fp8={fp8} {gran}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=100 + i)
    out = torch.full((B, T, H, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    ld = to_dev(lens)
    if fp8:
        qf, kf = q.float().numpy(), k.float().numpy()
        qs = quant.scales_from_amax(quant.group_amax(qf, lens, GRAN[gran]))
        ks = quant.scales_from_amax(quant.group_amax(kf, lens, GRAN[gran]))
        qc, kc = quant.quantize(qf, qs, GRAN[gran]), quant.quantize(kf, ks, GRAN[gran])
        wa.wa_encoder_attn_fp8qk(to_dev(qc), to_dev(qs), to_dev(kc), to_dev(ks), gran, to_dev(v), out=out,
                                 lens=ld, causal=causal, softmax_scale=0.125)
        want, mag = attn.dense_attention_fp8qk(qc, qs, kc, ks, GRAN[gran], v.float().numpy(), lens, causal,
                                               0.125, with_magnitude=True)
    else:
        wa.wa_encoder_attn(to_dev(q), to_dev(k), to_dev(v), out=out, lens=ld, causal=causal, softmax_scale=0.125)
        want, mag = attn.dense_attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), lens, causal,
                                         0.125, with_magnitude=True)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    mask = np.arange(T)[None, :] < lens[:, None]
    assert np.all(np.isnan(got[~mask])), "rows past a length were written"
    if mask.any():
        assert_close(torch.from_numpy(got[mask]), want[mask], f"random encoder #{i}", mag=mag[mask])


@pytest.mark.parametrize("i", range(10))
def test_decode_random(gpu, i):
    import whisper_attention_amd as wa
    g = _case_rng(2, i)
    B, H = int(g.integers(1, 41)), int(g.integers(1, 9))
    L = int(g.integers(1, 1601))
    lens = g.integers(0, L + 1, size=B).astype(np.int32)
    lens[g.integers(B)] = L
    gran = ["tensor", "head"][int(g.integers(2))]
    announce(f"random decode #{i}: B={B} H={H} L={L} gran={gran} (split when B*H < 640)")
    q, kc, vc, ks, vs, _ = workloads.decode_inputs(B, H, L, lens, gran, seed=200 + i, which="self")
    out = wa.wa_decode_attn(to_dev(q), to_dev(kc), to_dev(vc), to_dev(ks), to_dev(vs), to_dev(lens), gran, 0.125)
    torch.cuda.synchronize()
    want, mag = attn.decode_attention(q.float().numpy(), kc.numpy(), vc.numpy(), ks, vs, GRAN[gran], lens,
                                      0.125, with_magnitude=True)
    assert_close(out, want, f"random decode #{i}", mag=mag)


@pytest.mark.parametrize("i", range(6))
def test_quant_pair_random(gpu, i):
    import whisper_attention_amd as wa
    g = _case_rng(3, i)
    B, H = int(g.integers(1, 9)), int(g.integers(1, 25))
    T = int(g.integers(1, 300))
    L = int(g.integers(1, 320))
    lens = g.integers(0, T + 1, size=B).astype(np.int32)
    dst = g.integers(-5, L, size=B).astype(np.int32)
    gran = ["tensor", "head"][int(g.integers(2))]
    fmt = ["e4m3", "e5m2"][int(g.integers(2))]
    announce(f"random K/V quantize #{i}: B={B} H={H} T={T} L={L} {gran} {fmt}")
    k = workloads.bf16_normal((B, T, H, 64), 300 + i, 1, 0.02, 20.0)
    v = workloads.bf16_normal((B, T, H, 64), 300 + i, 2, 0.0, 20.0)
    kc = torch.full((B, H, L, 64), 0xA5, dtype=torch.uint8, device="cuda")
    vc = torch.full_like(kc, 0xA5)
    n = 1 if gran == "tensor" else H
    ks = torch.zeros(n, dtype=torch.float32, device="cuda")
    vs = torch.zeros_like(ks)
    wa.wa_kv_quant_fp8_kv(to_dev(k), to_dev(v), kc, vc, ks, vs, gran, fmt, lens=to_dev(lens), dst_start=to_dev(dst))
    torch.cuda.synchronize()
    f = quant.E4M3 if fmt == "e4m3" else quant.E5M2
    for name, x, c, s in (("K", k, kc, ks), ("V", v, vc, vs)):
        ref = np.full((B, H, L, 64), 0xA5, dtype=np.uint8)
        sw = quant.quantize_kv(x.float().numpy(), lens, dst, ref, GRAN[gran], f)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), sw.view(np.uint32)), f"{name} scales"
        got = c.cpu().numpy()
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{name}: {len(bad)} code mismatches, first {bad[:3].tolist()}"
