"""A decode step captured in a HIP graph (torch.cuda.graph over the wa_*
calls): per layer, the self-attention step with its append
(wa_decode_attn_append) and the cross-attention (wa_decode_attn).  The
calls allocate nothing, synchronise nothing and record no memset, so they
capture; every replay must equal the eager step, with eager work and
synchronisations between the replays, and every replay is checked against
the oracle: the appended codes bit for bit (a static-scale cache fill of
the step's token at slot lens[b] - 1), both attention outputs within the
parity bar."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attn, quant
from tests.gpu_helpers import announce, assert_close, to_dev

pytestmark = pytest.mark.gpu


def _layer_inputs(B, H, Ls, Lx, layers, seed):
    g = np.random.default_rng(seed)
    lay = []
    for layer in range(layers):
        lens_s = workloads.lens_uniform(B, 1, Ls, seed + layer)
        _, kc, vc, ks, vs, _ = workloads.decode_inputs(B, H, Ls, lens_s, "head", seed + layer, "self")
        _, xk, xv, xks, xvs, _ = workloads.decode_inputs(B, H, Lx, np.full(B, Lx), "tensor", seed + layer,
                                                         "cross")
        lay.append(dict(
            host=dict(kc=kc.numpy().copy(), vc=vc.numpy().copy(), ks=ks, vs=vs, lens_s=lens_s, xk=xk.numpy(),
                      xv=xv.numpy(), xks=xks, xvs=xvs),
            q=to_dev(workloads.bf16_normal((B, H, 64), seed + layer, 95)),
            qx=to_dev(workloads.bf16_normal((B, H, 64), seed + layer, 98)),
            kn=to_dev(workloads.bf16_normal((B, H, 64), seed + layer, 96)),
            vn=to_dev(workloads.bf16_normal((B, H, 64), seed + layer, 97)),
            kc=to_dev(kc), vc=to_dev(vc), ks=to_dev(ks), vs=to_dev(vs), lens_s=to_dev(lens_s),
            xk=to_dev(xk), xv=to_dev(xv), xks=to_dev(xks), xvs=to_dev(xvs),
            lens_x=to_dev(np.full(B, Lx, np.int32)),
            o_s=torch.empty((B, H, 64), dtype=torch.bfloat16, device="cuda"),
            o_x=torch.empty((B, H, 64), dtype=torch.bfloat16, device="cuda")))
    return lay


def _step(wa, lay, ws_s, ws_x):
    for L in lay:
        wa.wa_decode_attn_append(L["q"], L["kn"], L["vn"], L["kc"], L["vc"], L["ks"], L["vs"], L["lens_s"],
                                 "head", 0.125, out=L["o_s"], workspace=ws_s)
        # the layer's cross-attention (its query has its own seeded input
        # here, so that the oracle takes no input from the HIP path)
        wa.wa_decode_attn(L["qx"], L["xk"], L["xv"], L["xks"], L["xvs"], L["lens_x"], "tensor", 0.125,
                          out=L["o_x"], workspace=ws_x)


def _oracle(L):
    """Expected caches and outputs of one layer's step, from the host inputs:
    the step's token encoded with the stored per-head scales into slot
    lens[b] - 1 of the self cache, then both attentions over the caches."""
    h = L["host"]
    kc, vc = h["kc"].copy(), h["vc"].copy()
    n = np.asarray(h["lens_s"], np.int64)
    ones = (n > 0).astype(np.int64)
    dst = np.maximum(n - 1, 0)
    quant.fill_cache(L["kn"].float().cpu().numpy()[:, None], ones, dst, kc, h["ks"], quant.PER_HEAD)
    quant.fill_cache(L["vn"].float().cpu().numpy()[:, None], ones, dst, vc, h["vs"], quant.PER_HEAD)
    o_s, m_s = attn.decode_attention(L["q"].float().cpu().numpy(), kc, vc, h["ks"], h["vs"], quant.PER_HEAD, n,
                                     0.125, with_magnitude=True)
    B = n.shape[0]
    o_x, m_x = attn.decode_attention(L["qx"].float().cpu().numpy(), h["xk"], h["xv"], h["xks"], h["xvs"],
                                     quant.PER_TENSOR, np.full(B, h["xk"].shape[2]), 0.125, with_magnitude=True)
    return kc, vc, (o_s, m_s), (o_x, m_x)


@pytest.mark.parametrize("B,H", [(64, 20), (1, 20)])
def test_captured_decode_step_equals_eager(gpu, B, H):
    import whisper_attention_amd as wa
    announce(f"decode step in a HIP graph: B={B} H={H}, 4 layers")
    Ls, Lx = 448, 1500
    lay = _layer_inputs(B, H, Ls, Lx, 4, 11)
    ws_s = torch.zeros(max(16, wa.wa_decode_attn_workspace_size(B, H, Ls)), dtype=torch.uint8, device="cuda")
    ws_x = torch.zeros(max(16, wa.wa_decode_attn_workspace_size(B, H, Lx)), dtype=torch.uint8, device="cuda")
    _step(wa, lay, ws_s, ws_x)                  # eager reference (also warms up)
    torch.cuda.synchronize()
    ref = [(L["o_s"].clone(), L["o_x"].clone(), L["kc"].clone(), L["vc"].clone()) for L in lay]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(wa, lay, ws_s, ws_x)             # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        _step(wa, lay, ws_s, ws_x)
    want = [_oracle(L) for L in lay]
    for replay in range(3):
        for L in lay:                            # eager work between replays
            L["o_s"].fill_(float("nan"))
            L["o_x"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, L in enumerate(lay):
            o_s, o_x, kc, vc = ref[i]
            assert torch.equal(L["o_s"].view(torch.int16), o_s.view(torch.int16)), (replay, i, "self")
            assert torch.equal(L["o_x"].view(torch.int16), o_x.view(torch.int16)), (replay, i, "cross")
            assert torch.equal(L["kc"], kc) and torch.equal(L["vc"], vc), (replay, i, "cache")
            wkc, wvc, (ws_o, ws_m), (wx_o, wx_m) = want[i]
            assert np.array_equal(L["kc"].cpu().numpy(), wkc), (replay, i, "K cache vs oracle")
            assert np.array_equal(L["vc"].cpu().numpy(), wvc), (replay, i, "V cache vs oracle")
            assert_close(L["o_s"], ws_o, f"graph replay {replay} layer {i} self B={B}", mag=ws_m)
            assert_close(L["o_x"], wx_o, f"graph replay {replay} layer {i} cross B={B}", mag=wx_m)


def test_captured_prompt_step_equals_eager(gpu):
    """The prompt side captured in one graph: the K/V cache fill with dynamic
    per-head scales (wa_kv_quant_fp8_kv: amax, scale and encode kernels), the
    causal prefill attention and the prompt cross-attention against encoder
    frames (wa_cross_attn), then the encoder attention.  Three replays, with
    eager work between them, equal the eager pass bit for bit (outputs,
    codes and scales) and the oracle: codes and scales bit for bit, the
    attention outputs within the parity bar."""
    import whisper_attention_amd as wa
    B, H, T, Tk, L = 16, 20, 224, 1500, 256
    announce(f"prompt step in a HIP graph: B={B} H={H} T={T} frames={Tk}")
    lens = to_dev(workloads.lens_uniform(B, 4, T, 21))
    q = to_dev(workloads.bf16_normal((B, T, H, 64), 21, 1))
    k = to_dev(workloads.bf16_normal((B, T, H, 64), 21, 2, 0.01, 20.0))
    v = to_dev(workloads.bf16_normal((B, T, H, 64), 21, 3, 0.01, 20.0))
    qx, kx, vx = (to_dev(t) for t in workloads.cross_inputs(2, H, T, Tk, seed=22))
    kx, vx = kx[:1].expand(B, Tk, H, 64), vx[:1].expand(B, Tk, H, 64)   # one chunk's frames for every prompt
    qe, ke, ve = (to_dev(t) for t in workloads.encoder_inputs(1, H, Tk, seed=23))
    kc = torch.zeros((B, H, L, 64), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    ks = torch.zeros(H, dtype=torch.float32, device="cuda")
    vs = torch.zeros_like(ks)
    half = wa.wa_kv_quant_fp8_workspace_size(B, H, "head")
    ws = torch.zeros(2 * half, dtype=torch.uint8, device="cuda")
    o_p, o_x = torch.empty_like(q), torch.empty_like(q)
    o_e = torch.empty_like(qe)

    def step():
        wa.wa_kv_quant_fp8_kv(k, v, kc, vc, ks, vs, "head", lens=lens, workspace=ws)
        wa.wa_encoder_attn(q, k, v, out=o_p, lens=lens, causal=True, softmax_scale=0.125)
        wa.wa_cross_attn(q, kx, vx, out=o_x, q_lens=lens, softmax_scale=0.125)
        wa.wa_encoder_attn(qe, ke, ve, out=o_e, softmax_scale=0.125)

    outs = (o_p, o_x, o_e, kc, vc, ks, vs)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    # the oracle, from the host inputs
    lh = lens.cpu().numpy()
    qh, kh, vh = (t.float().cpu().numpy() for t in (q, k, v))
    wkc = np.zeros((B, H, L, 64), np.uint8)
    wvc = np.zeros_like(wkc)
    zero = np.zeros(B, np.int64)
    wks = quant.quantize_kv(kh, lh, zero, wkc, quant.PER_HEAD)
    wvs = quant.quantize_kv(vh, lh, zero, wvc, quant.PER_HEAD)
    w_p, m_p = attn.dense_attention(qh, kh, vh, lh, True, 0.125, with_magnitude=True)
    w_x, m_x = attn.cross_attention(qh, kx.float().cpu().numpy(), vx.float().cpu().numpy(), lh,
                                    np.full(B, Tk), 0.125, with_magnitude=True)
    w_e, m_e = attn.dense_attention(qe.float().cpu().numpy(), ke.float().cpu().numpy(), ve.float().cpu().numpy(),
                                    [Tk], False, 0.125, with_magnitude=True)
    valid = np.arange(T)[None, :] < lh[:, None]
    for replay in range(3):
        for t in outs:                          # eager work between replays
            t.zero_()
        # the partials need no initialisation; the counters at the start of
        # each tensor's half are zero, as every call leaves them
        for part in (ws[256:half], ws[half + 256:]):
            part.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert not ws[:256].any() and not ws[half:half + 256].any(), (replay, "counters not left at zero")
        for i, (t, r) in enumerate(zip(outs, ref)):
            a = t.view(torch.uint8) if t.dtype != torch.uint8 else t
            b = r.view(torch.uint8) if r.dtype != torch.uint8 else r
            assert torch.equal(a, b), (replay, i)
        assert np.array_equal(kc.cpu().numpy(), wkc) and np.array_equal(vc.cpu().numpy(), wvc), replay
        assert np.array_equal(ks.cpu().numpy().view(np.uint32), wks.view(np.uint32)), replay
        assert np.array_equal(vs.cpu().numpy().view(np.uint32), wvs.view(np.uint32)), replay
        gp, gx = o_p.float().cpu().numpy(), o_x.float().cpu().numpy()
        assert_close(torch.from_numpy(gp[valid]), w_p[valid], f"graph replay {replay} prefill", mag=m_p[valid])
        assert_close(torch.from_numpy(gx[valid]), w_x[valid], f"graph replay {replay} prompt cross",
                     mag=m_x[valid])
        assert_close(o_e, w_e, f"graph replay {replay} encoder", mag=m_e)
