"""Seeded synthetic inputs for the Whisper attention hot path.

Shared by the tests, the benchmark and the smoke check, and by both sides of
every parity comparison (the HIP library and the CPU oracle).  It holds none
of the method's arithmetic: only random draws, the bf16 rounding of those
draws, and the shapes of the workloads.

Shapes follow the Whisper workloads the pages describe: a 30-second audio
chunk is the encoder's unit (whisper-blaze 0.1.8, "Batch Transcription");
with Whisper's 20 ms encoder frame that is 1500 frames; large-v3 has 20 heads
of width 64; the decoder's cache holds at most 448 tokens; long files are cut
into thirty 30-s chunks per 15 minutes and all chunks of several files run as
one batch (whisper-blaze, "Batch Transcription" and "VRAM usage guide").

Every tensor draws from its own stream, ``numpy.random.SeedSequence([seed,
tensor_id])`` with PCG64, so one tensor can be regenerated without the
others.  bf16 values are fp32 samples rounded to nearest even by torch.
"""
import numpy as np
import torch

HEAD_DIM = 64
ENC_FRAMES = 1500          # 30 s of audio at 50 encoder frames per second
DEC_MAX_TOKENS = 448       # Whisper's decoder context

# Fixed tensor ids, so each stream is stable across code changes.
TID_Q, TID_K, TID_V = 1, 2, 3
TID_LENS = 4
TID_DQ = 5
TID_XK_CODES, TID_XV_CODES = 6, 7          # cross-attention cache codes
TID_SK_CODES, TID_SV_CODES = 8, 9          # self-attention cache codes
TID_XK_SCALE, TID_XV_SCALE = 10, 11
TID_SK_SCALE, TID_SV_SCALE = 12, 13
TID_KV_K, TID_KV_V = 14, 15                # bf16 K/V to be quantized
TID_XK_BF16, TID_XV_BF16 = 16, 17          # bf16 cross-attention K/V (encoder frames)


def rng(seed, tid):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid])))


def bf16_normal(shape, seed, tid, outlier_p=0.0, outlier_mult=20.0):
    """bf16 CPU tensor of N(0,1) samples; with probability ``outlier_p`` an
    element is multiplied by ``outlier_mult`` before rounding to bf16."""
    g = rng(seed, tid)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if outlier_p > 0:
        mask = g.random(size=shape, dtype=np.float32) < outlier_p
        x = np.where(mask, x * np.float32(outlier_mult), x)
    return torch.from_numpy(x).to(torch.bfloat16)


def lens_uniform(B, lo, hi, seed, tid=TID_LENS):
    """int32 lengths uniform on the integers [lo, hi]."""
    return rng(seed, tid).integers(lo, hi + 1, size=B).astype(np.int32)


def lens_zipf(B, a, cap, seed, tid=TID_LENS):
    """int32 lengths min(Zipf(a), cap)."""
    return np.minimum(rng(seed, tid).zipf(a, size=B), cap).astype(np.int32)


def _fp8_byte_map():
    """256-entry map from a uniform random byte to a synthetic E4M3 code.

    Bit 0 is the sign, bits 1-3 the mantissa, and the top four bits pick how
    many binades below the top one the exponent field sits: 0 for half of
    them, 1 for a quarter, 2 for an eighth, 3 and 4 for a sixteenth each.
    Exponent 15 with mantissa 7 (NaN) becomes mantissa 6.
    """
    drop = [0] * 8 + [1] * 4 + [2] * 2 + [3] + [4]
    out = np.zeros(256, dtype=np.uint8)
    for r in range(256):
        sign, m, e = r & 1, (r >> 1) & 7, 15 - drop[r >> 4]
        if e == 15 and m == 7:
            m = 6
        out[r] = (sign << 7) | (e << 3) | m
    return out


_FP8_BYTE_MAP = _fp8_byte_map()


def fp8_codes(shape, seed, tid):
    """Synthetic E4M3 cache bytes shaped like a quantized bell curve (uint8 CPU tensor).

    Uniform random bytes sent through a fixed 256-entry map: magnitudes
    concentrate in the top binades as codes of a quantized Gaussian do, and
    no NaN pattern occurs.  Used where a cache is an input in its own right;
    codes produced by quantizing bf16 data come from the quantize step.
    """
    r = rng(seed, tid).integers(0, 256, size=shape, dtype=np.uint8)
    return torch.from_numpy(_FP8_BYTE_MAP[r])


def scales_uniform(n, seed, tid, lo=2.0 / 448, hi=6.0 / 448):
    """float32 dequantization scales, uniform on [lo, hi] (amax 2..6 over 448)."""
    return rng(seed, tid).uniform(lo, hi, size=n).astype(np.float32)


# ---------------------------------------------------------------------------
# The five workloads.  Activations are [B][T][H][D]; caches are [B][H][L][D].
# ---------------------------------------------------------------------------

CONFIGS = {
    # one chunk, 6 heads: encoder at T=1500; one decode step against 1500
    # cross frames and a 64-token self cache, per-tensor scales
    "tiny": dict(B=1, H=6, T=ENC_FRAMES, self_len=64, gran="tensor"),
    # large-v3 encoder: 16 chunks, 20 heads
    "enc_l3": dict(B=16, H=20, T=ENC_FRAMES),
    # large-v3 decode step: 64 sequences, self lengths U[1,448], per-tensor
    "dec_l3": dict(B=64, H=20, cross_len=ENC_FRAMES, self_lo=1, self_hi=DEC_MAX_TOKENS,
                   gran="tensor"),
    # decoder prompt prefill + cache fill: lengths U[4,224], 1% outliers x20
    "prefill": dict(B=128, H=20, T=224, lo=4, hi=224, outlier_p=0.01, outlier_mult=20.0,
                    gran="head"),
    # encoder at the shorter windows: 10-s (500 frames) and 15-s (750
    # frames) chunks, batches sized to the same B*T^2 work as enc_l3
    # decoder prompt prefill attending to the 1500 encoder frames:
    # prompt lengths U[4,224], bf16 K/V with 1% outliers x20
    "prefill_cross": dict(B=128, H=20, T=224, lo=4, hi=224, T_k=ENC_FRAMES, outlier_p=0.01,
                          outlier_mult=20.0),
    "enc_10s": dict(B=144, H=20, T=500),
    "enc_15s": dict(B=64, H=20, T=750),
    # long audio: 256 chunks (thirty per 15-minute file), Zipf(1.2) self
    # lengths capped at 448, per-head scales
    "long": dict(B=256, H=20, cross_len=ENC_FRAMES, zipf_a=1.2, cap=DEC_MAX_TOKENS,
                 gran="head"),
}


def encoder_inputs(B, H, T, seed=0):
    """bf16 Q, K, V [B][T][H][64], each N(0,1)."""
    shape = (B, T, H, HEAD_DIM)
    return (bf16_normal(shape, seed, TID_Q), bf16_normal(shape, seed, TID_K),
            bf16_normal(shape, seed, TID_V))


def prefill_inputs(B, H, T, lo, hi, outlier_p, outlier_mult, seed=0):
    """bf16 Q, K, V [B][T][H][64] with outliers in K and V, and lengths U[lo, hi]."""
    shape = (B, T, H, HEAD_DIM)
    q = bf16_normal(shape, seed, TID_Q)
    k = bf16_normal(shape, seed, TID_K, outlier_p, outlier_mult)
    v = bf16_normal(shape, seed, TID_V, outlier_p, outlier_mult)
    return q, k, v, lens_uniform(B, lo, hi, seed)


def cross_inputs(B, H, Tq, Tk, outlier_p=0.0, outlier_mult=20.0, seed=0):
    """bf16 Q [B][Tq][H][64] (N(0,1)) and K, V [B][Tk][H][64] (N(0,1) with
    outliers)."""
    q = bf16_normal((B, Tq, H, HEAD_DIM), seed, TID_Q)
    k = bf16_normal((B, Tk, H, HEAD_DIM), seed, TID_XK_BF16, outlier_p, outlier_mult)
    v = bf16_normal((B, Tk, H, HEAD_DIM), seed, TID_XV_BF16, outlier_p, outlier_mult)
    return q, k, v


def decode_inputs(B, H, L, lens, gran, seed=0, which="self"):
    """One decode step against one cache.

    Returns q bf16 [B][H][64], K/V codes uint8 [B][H][L][64] and float32
    scales ([1] or [H]).  ``which`` selects independent streams for the
    self- and the cross-attention cache.
    """
    tk, tv, sk, sv = ((TID_SK_CODES, TID_SV_CODES, TID_SK_SCALE, TID_SV_SCALE)
                      if which == "self" else
                      (TID_XK_CODES, TID_XV_CODES, TID_XK_SCALE, TID_XV_SCALE))
    n = 1 if gran == "tensor" else H
    q = bf16_normal((B, H, HEAD_DIM), seed, TID_DQ)
    kc = fp8_codes((B, H, L, HEAD_DIM), seed, tk)
    vc = fp8_codes((B, H, L, HEAD_DIM), seed, tv)
    return q, kc, vc, scales_uniform(n, seed, sk), scales_uniform(n, seed, sv), \
        np.asarray(lens, dtype=np.int32)
