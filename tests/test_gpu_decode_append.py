"""GPU parity of wa_decode_attn_append: the new token's K/V codes written to
slot lens[b] - 1 bit-exact (every other slot untouched), and the output
within max-abs 2e-2 / mean-abs 2e-3 of the oracle's attention over the
updated cache."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attn, quant
from tests.gpu_helpers import announce, assert_close, to_dev

pytestmark = pytest.mark.gpu

GUARD_K, GUARD_V = 0x7F, 0xFF      # NaN codes: never read past a length


def _case(B, H, L, lens, gran, seed, Lbuf=None):
    """Caches of capacity Lbuf >= L holding valid codes below lens[b]-1 and
    NaN guard codes at and beyond it; returns host arrays."""
    Lbuf = L if Lbuf is None else Lbuf
    q, kc, vc, ks, vs, lens = workloads.decode_inputs(B, H, L, lens, gran, seed, "self")
    kcache = np.full((B, H, Lbuf, 64), GUARD_K, np.uint8)
    vcache = np.full((B, H, Lbuf, 64), GUARD_V, np.uint8)
    for b in range(B):
        n = min(int(lens[b]), L)
        kcache[b, :, :max(n - 1, 0)] = kc.numpy()[b, :, :max(n - 1, 0)]
        vcache[b, :, :max(n - 1, 0)] = vc.numpy()[b, :, :max(n - 1, 0)]
    kn = workloads.bf16_normal((B, H, 64), seed, 90, 0.02, 20.0)
    vn = workloads.bf16_normal((B, H, 64), seed, 91, 0.02, 20.0)
    return q, kn, vn, kcache, vcache, ks, vs, np.asarray(lens, np.int32)


def _oracle(q, kn, vn, kcache, vcache, ks, vs, lens, gran, L):
    g = quant.PER_TENSOR if gran == "tensor" else quant.PER_HEAD
    kc, vc = kcache.copy(), vcache.copy()
    n = np.minimum(lens, L)
    dst = np.maximum(n - 1, 0)
    ones = (n > 0).astype(np.int64)          # one token per sequence, none when n == 0
    quant.fill_cache(kn.float().numpy()[:, None], ones, dst, kc, ks, g)
    quant.fill_cache(vn.float().numpy()[:, None], ones, dst, vc, vs, g)
    out, mag = attn.decode_attention(q.float().numpy(), kc[:, :, :L], vc[:, :, :L], ks, vs, g, n, 0.125,
                                     with_magnitude=True)
    return kc, vc, out, mag


def _gpu(wa, q, kn, vn, kcache, vcache, ks, vs, lens, gran, L):
    kd, vd = to_dev(kcache), to_dev(vcache)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    wa.wa_decode_attn_append(to_dev(q), to_dev(kn), to_dev(vn), kd[:, :, :L], vd[:, :, :L], to_dev(ks),
                             to_dev(vs), to_dev(lens), gran, 0.125, out=out)
    torch.cuda.synchronize()
    return kd.cpu().numpy(), vd.cpu().numpy(), out


@pytest.mark.parametrize("gran", ["tensor", "head"])
@pytest.mark.parametrize("B,H,L,Lbuf", [(64, 20, 448, 448), (5, 4, 1500, 1500), (3, 2, 300, 320),
                                        (700, 1, 64, 64)])
def test_append_then_attend(gpu, B, H, L, Lbuf, gran):
    import whisper_attention_amd as wa
    announce(f"decode append B={B} H={H} L={L} buffer {Lbuf} {gran}")
    g = np.random.default_rng(B + L)
    lens = g.integers(1, L + 1, size=B)
    lens[0] = L
    if B > 1:
        lens[1] = 1
    if B > 2:
        lens[2] = 0
    q, kn, vn, kc, vc, ks, vs, lens = _case(B, H, L, lens, gran, 3, Lbuf)
    wk, wv, want, mag = _oracle(q, kn, vn, kc, vc, ks, vs, lens, gran, L)
    gk, gv, got = _gpu(wa, q, kn, vn, kc, vc, ks, vs, lens, gran, L)
    bad = np.argwhere(gk != wk)
    assert bad.size == 0, f"K cache differs at {bad[:4].tolist()}"
    assert np.array_equal(gv, wv), "V cache differs"
    assert_close(got, want, f"append B={B} H={H} L={L} {gran}", mag=mag)
    assert torch.all(got[torch.as_tensor(np.asarray(lens) == 0, device="cuda")].float() == 0)


def test_append_steps_match_quantize_then_decode(gpu):
    """Three decode steps in a row: append + attend in one call against the
    two-call path (wa_kv_quant_fp8 with the stored scale at slot n-1, then
    wa_decode_attn): codes bit for bit; outputs within the parity bar (the
    new row is summed in a different order)."""
    import whisper_attention_amd as wa
    announce("decode append, three steps vs quantize + decode")
    B, H, L = 8, 20, 448
    lens0 = workloads.lens_uniform(B, 1, L - 3, 4)
    q, kn, vn, kc, vc, ks, vs, lens = _case(B, H, L, lens0, "head", 4)
    k1, v1 = to_dev(kc), to_dev(vc)
    k2, v2 = to_dev(kc), to_dev(vc)
    ksd, vsd = to_dev(ks), to_dev(vs)
    for step in range(3):
        n = torch.as_tensor(lens + step, device="cuda")
        qs = to_dev(workloads.bf16_normal((B, H, 64), step, 92))
        kns = to_dev(workloads.bf16_normal((B, H, 64), step, 93))
        vns = to_dev(workloads.bf16_normal((B, H, 64), step, 94))
        a = wa.wa_decode_attn_append(qs, kns, vns, k1, v1, ksd, vsd, n, "head", 0.125)
        one = torch.ones(B, dtype=torch.int32, device="cuda")
        wa.wa_kv_quant_fp8(kns[:, None], k2, ksd, "head", lens=one, dst_start=n - 1, compute_scale=False)
        wa.wa_kv_quant_fp8(vns[:, None], v2, vsd, "head", lens=one, dst_start=n - 1, compute_scale=False)
        b = wa.wa_decode_attn(qs, k2, v2, ksd, vsd, n, "head", 0.125)
        torch.cuda.synchronize()
        assert torch.equal(k1, k2) and torch.equal(v1, v2), f"step {step}: caches differ"
        assert_close(a, b.double().cpu().numpy(), f"append step {step} vs quantize + decode")
