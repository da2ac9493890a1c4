"""Plain CPU oracle for the Whisper attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this package: it is used by ``tests/``, by the smoke check in
``__graft_entry__.py`` and by the ``cpu_baseline`` leg of ``bench.py``.
It shares no code with the HIP library (``whisper_attention_amd``); the
only thing both sides see is the seeded input generator in ``workloads.py``,
which holds none of the method's arithmetic.

What it computes, and where the pages define it:

* ``e4m3``  -- the OCP float8 E4M3 ("E4M3FN") codec: exact decode of all
  256 codes and a round-to-nearest-even, saturating encode.  The format is
  named by whisper-blaze 0.1.8 (PyPI page, feature list: "FP8 ... E4M3" and
  "Direct Kernel API": ``quantise_e4m3``); the HF blog post "Blazingly fast
  whisper transcriptions with Inference Endpoints" (section "Inference
  Stack") fixes that the KV cache is stored in one-byte float8.
* ``e5m2``  -- the OCP float8 E5M2 codec, the second FP8 format that
  whisper-blaze's feature list names: exact decode of all 256 codes and a
  round-to-nearest-even encode that saturates at 57344.
* ``quant`` -- dynamic KV quantization: abs-max per scale group, the
  dequantization multiplier ``scale = amax / 448`` (E4M3; 57344 for E5M2)
  and the codes ``FMT(x / scale)``, and the dequantise back to bf16;
  whisper-blaze "Direct Kernel API" (quantise returns codes plus a scale;
  dequantise takes codes and that scale) and its feature list ("per-tensor
  scaling"); HF blog "Inference Stack" ("dynamically quantizing
  activations" for the KV cache).
* ``attn``  -- softmax attention: dense non-causal (encoder
  self-attention), causal and ragged (decoder prompt prefill), and one
  query token against an fp8 cache (decoder self- and cross-attention),
  plus the split-key partial/merge identity.  whisper-blaze "Direct Kernel
  API" (encoder_self_attn with no mask, decoder_self_attn causal,
  decoder_cross_attn with no mask); "Unlocking the power of OpenAI's
  Whisper", section 3 (encoder self-attention; decoder self- and
  cross-attention).

Precision: the quantize step decides integer codes, so it runs in IEEE fp32
exactly as the kernel does (the pages fix no other precision for it); the
attention functions run in float64 on the exact input values, which is the
plain definition with rounding error far below the parity tolerance.
"""
