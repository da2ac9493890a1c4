"""Softmax attention -- oracle side (test infrastructure only).

The three attentions of the Whisper hot path, as whisper-blaze 0.1.8 (PyPI
page, "Direct Kernel API") names them -- encoder self-attention with no
mask, decoder self-attention with a causal mask, decoder cross-attention with
no mask -- and as "Unlocking the power of OpenAI's Whisper", section 3,
places them (the encoder attends over the audio frames; the decoder attends
over its previous tokens and over the encoded audio).

The pages print no formula; the plain reading is scaled dot-product softmax
attention, per sequence b and head h, for a query row i:

    s_j = softmax_scale * sum_d Q[i,d] K[j,d]        over the allowed keys j
    p_j = exp(s_j - max_j s_j)
    O[i] = sum_j p_j V[j] / sum_j p_j

Allowed keys: j < lens[b] (ragged, non-causal) and additionally j <= i when
causal.  Rows i >= lens[b] have no output (returned as NaN here).  One decode
query sits at the last cached position, so it sees every slot j < lens[b];
a sequence of length 0 gives a zero row.  Decode attention reads K and V
from the fp8 cache, dequantized as ``decode(code) * scale``.

Everything runs in float64 on the exact input values: no tiling, no online
rescaling, two passes over the scores.
"""
import numpy as np

from . import quant


def dense_attention(q, k, v, lens, causal, softmax_scale, with_magnitude=False):
    """q, k, v: [B][T][H][D] (bf16 values as float) -> O float64 [B][T][H][D].

    Rows i >= lens[b] are NaN.  With ``with_magnitude`` also returns
    sum_j p_j |V[j]| / sum_j p_j, the size of the terms each output sums
    (rounding the weights p by a relative e moves O by at most e times it).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, D = q.shape
    out = np.full((B, T, H, D), np.nan, dtype=np.float64)
    mag = np.full((B, T, H, D), np.nan, dtype=np.float64) if with_magnitude else None
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(H):
            qb = q[b, :n, h, :]                  # [n][D]
            kb = k[b, :n, h, :]
            vb = v[b, :n, h, :]
            s = softmax_scale * (qb @ kb.T)      # [n queries][n keys]
            if causal:
                s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            out[b, :n, h, :] = (p @ vb) / p.sum(axis=1, keepdims=True)
            if with_magnitude:
                mag[b, :n, h, :] = (p @ np.abs(vb)) / p.sum(axis=1, keepdims=True)
    return (out, mag) if with_magnitude else out


def cross_attention(q, k, v, q_lens, k_lens, softmax_scale, with_magnitude=False):
    """Decoder cross-attention with a multi-token query (a prompt attending to
    the encoded audio): whisper-blaze's decoder_cross_attn, which masks nothing
    (PyPI page, "Direct Kernel API"), with the query and the keys of
    different lengths ("Unlocking the power of OpenAI's Whisper", section 3:
    the decoder attends over the encoder's output).

    q: [B][Tq][H][D]; k, v: [B][Tk][H][D].  Query row i < q_lens[b] attends
    to every key j < k_lens[b]; other rows are NaN, and a row with no key
    (k_lens[b] = 0) is zero.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Tq, H, D = q.shape
    out = np.full((B, Tq, H, D), np.nan, dtype=np.float64)
    mag = np.full((B, Tq, H, D), np.nan, dtype=np.float64) if with_magnitude else None
    for b in range(B):
        nq, nk = int(q_lens[b]), int(k_lens[b])
        if nq == 0:
            continue
        if nk == 0:
            out[b, :nq] = 0.0
            if with_magnitude:
                mag[b, :nq] = 0.0
            continue
        for h in range(H):
            s = softmax_scale * (q[b, :nq, h, :] @ k[b, :nk, h, :].T)   # [nq][nk]
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, :nq, h, :] = (p @ v[b, :nk, h, :]) / p.sum(axis=1, keepdims=True)
            if with_magnitude:
                mag[b, :nq, h, :] = (p @ np.abs(v[b, :nk, h, :])) / p.sum(axis=1, keepdims=True)
    return (out, mag) if with_magnitude else out


def dense_attention_fp8qk(q_codes, q_scale, k_codes, k_scale, gran, v, lens, causal, softmax_scale,
                          with_magnitude=False):
    """Dense attention with Q and K given as E4M3 codes and dequantization scales.

    The ``aggressive_fp8`` preset of whisper-blaze 0.1.8 (PyPI page,
    "Precision Presets": FP8 everywhere) read for attention as Q and K stored
    in float8 E4M3 with the quantize step's scales, V and the output in
    bf16.  The attention is exactly ``dense_attention`` over the dequantized
    values ``decode(code) * scale[g]`` (g = 0, or the head with per-head
    scales).  q_codes, k_codes: uint8 [B][T][H][D]; v: [B][T][H][D].
    """
    qh = quant.dequantize(q_codes, q_scale, gran, head_axis=2)
    kh = quant.dequantize(k_codes, k_scale, gran, head_axis=2)
    return dense_attention(qh, kh, v, lens, causal, softmax_scale, with_magnitude)


def decode_attention_dequant(q, khat, vhat, lens, softmax_scale, with_magnitude=False):
    """One query per (b, h) against already-dequantized keys and values.

    q: [B][H][D]; khat, vhat: [B][H][L][D] float; lens: [B].  -> [B][H][D] float64
    (plus sum_j p_j |V^_j| / sum_j p_j with ``with_magnitude``).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, D = q.shape
    out = np.zeros((B, H, D), dtype=np.float64)
    mag = np.zeros((B, H, D), dtype=np.float64)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(H):
            kb = np.asarray(khat[b, h, :n, :], dtype=np.float64)
            vb = np.asarray(vhat[b, h, :n, :], dtype=np.float64)
            s = softmax_scale * (kb @ q[b, h])   # [n]
            p = np.exp(s - s.max())
            out[b, h] = (p @ vb) / p.sum()
            mag[b, h] = (p @ np.abs(vb)) / p.sum()
    return (out, mag) if with_magnitude else out


def decode_attention(q, k_cache, v_cache, k_scale, v_scale, gran, lens, softmax_scale,
                     with_magnitude=False):
    """One query token per (b, h) against the fp8 KV cache.

    k_cache, v_cache: uint8 codes [B][H][L][D]; k_scale, v_scale: float32 [1]
    or [H] (``gran``); lens: [B].  Keys and values are dequantized explicitly
    as ``decode(code) * scale`` before the softmax.  -> [B][H][D] float64.
    """
    khat = quant.dequantize(k_cache, k_scale, gran, head_axis=1)
    vhat = quant.dequantize(v_cache, v_scale, gran, head_axis=1)
    return decode_attention_dequant(q, khat, vhat, lens, softmax_scale, with_magnitude)


def decode_partial(q, kb, vb, softmax_scale):
    """Partial softmax state over one chunk of keys for a single query.

    q: [D]; kb, vb: [n][D] with n >= 1.  Returns (m, l, o_tilde): the chunk's
    score maximum, sum of exp(s - m) and the unnormalised sum of
    exp(s - m) * V.
    """
    s = softmax_scale * (np.asarray(kb, dtype=np.float64) @ np.asarray(q, dtype=np.float64))
    m = s.max()
    p = np.exp(s - m)
    return m, p.sum(), p @ np.asarray(vb, dtype=np.float64)


def merge_partials(ms, ls, os_):
    """Combine chunk partials (m_i, l_i, o_i) into the softmax output.

    With M = max_i m_i:  O = sum_i exp(m_i - M) o_i / sum_i exp(m_i - M) l_i.
    The pages are silent on split-key evaluation (whisper-blaze only names
    "Flash Attention 3"); this is the standard rescaling identity.
    """
    ms = np.asarray(ms, dtype=np.float64)
    M = ms.max()
    w = np.exp(ms - M)
    num = (w[:, None] * np.asarray(os_, dtype=np.float64)).sum(axis=0)
    den = (w * np.asarray(ls, dtype=np.float64)).sum()
    return num / den
