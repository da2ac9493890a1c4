"""A decode step captured in a HIP graph (torch.cuda.graph over the wa_*
calls): per layer, the self-attention step with its append
(wa_decode_attn_append) and the cross-attention (wa_decode_attn).  The
calls allocate nothing, synchronise nothing and record no memset, so they
capture; every replay must equal the eager step, with eager work and
synchronisations between the replays."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import announce, to_dev

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
            q=to_dev(workloads.bf16_normal((B, H, 64), seed + layer, 95)),
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
        # the layer's cross-attention query depends on the self-attention
        # output in the model; here it reuses it as the query
        wa.wa_decode_attn(L["o_s"], L["xk"], L["xv"], L["xks"], L["xvs"], L["lens_x"], "tensor", 0.125,
                          out=L["o_x"], workspace=ws_x)


@pytest.mark.parametrize("B,H", [(64, 20), (1, 20)])
def test_captured_decode_step_equals_eager(gpu, B, H):
    import whisper_attention_amd as wa
    announce(f"decode step in a HIP graph: B={B} H={H}, 4 layers")
    Ls, Lx = 448, 1500
    lay = _layer_inputs(B, H, Ls, Lx, 4, 11)
    ws_s = torch.empty(max(16, wa.wa_decode_attn_workspace_size(B, H, Ls)), dtype=torch.uint8, device="cuda")
    ws_x = torch.empty(max(16, wa.wa_decode_attn_workspace_size(B, H, Lx)), dtype=torch.uint8, device="cuda")
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
