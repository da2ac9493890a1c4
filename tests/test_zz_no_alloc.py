"""wa_decode_attn_noalloc (no workspace, a static device scratch array)
against wa_decode_attn through the C ABI: two calls in a row, the second
with a smaller input, each bit for bit equal to the workspace entry point
on the same inputs and within the parity bar of the oracle.  Both calls
split the keys, so both go through the scratch array and the merge."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attn, quant
from tests.gpu_helpers import announce, assert_close, to_dev

pytestmark = pytest.mark.gpu


def test_noalloc_decode_equals_workspace_entry_point(gpu):
    import whisper_attention_amd as wa
    cases = [(8, 20, 1500, "tensor", 41), (2, 6, 300, "head", 42)]
    for i, (B, H, L, gran, seed) in enumerate(cases):
        need = wa.wa_decode_attn_workspace_size(B, H, L)
        announce(f"noalloc decode call {i}: B={B} H={H} L={L} {gran}, partials {need} bytes")
        assert 0 < need <= wa.WA_DECODE_NOALLOC_SCRATCH_BYTES
        lens = workloads.lens_uniform(B, 1, L, seed)
        lens[0] = L
        q, kc, vc, ks, vs, lens = workloads.decode_inputs(B, H, L, lens, gran, seed, "cross")
        qd, kd, vd, ksd, vsd, ld = (to_dev(t) for t in (q, kc, vc, ks, vs, lens))
        out_n = torch.full((B, H, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
        wa.wa_decode_attn_noalloc(qd, kd, vd, ksd, vsd, ld, gran, out_n)
        out_w = wa.wa_decode_attn(qd, kd, vd, ksd, vsd, ld, gran)
        torch.cuda.synchronize()
        assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16)), f"call {i}: differs from wa_decode_attn"
        g = quant.PER_TENSOR if gran == "tensor" else quant.PER_HEAD
        want, mag = attn.decode_attention(q.float().numpy(), kc.numpy(), vc.numpy(), ks, vs, g, lens, 0.125,
                                          with_magnitude=True)
        assert_close(out_n, want, f"noalloc decode call {i}", mag=mag)
