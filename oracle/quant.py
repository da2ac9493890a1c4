"""Dynamic bf16 -> float8 KV quantization -- oracle side (test infrastructure only).

Follows the HF blog "Blazingly fast whisper transcriptions with Inference
Endpoints", section "Inference Stack" (activations are quantized dynamically
and the KV cache stores one byte per element while compute stays bf16), and
whisper-blaze 0.1.8 (PyPI page): the feature list ("FP8 quantize/dequantize
with per-tensor scaling") and "Direct Kernel API" (``quantise_e4m3`` returns
the codes and a scale; ``dequantise_e4m3`` takes the codes and that scale).

Readings where the pages are silent:

* the format is E4M3 unless E5M2 is asked for (the feature list names both
  for its FP8 GEMMs; the quantize call it shows is the E4M3 one);
* the scale is the dequantization multiplier, ``x ~= decode(code) * scale``,
  chosen so the group's largest magnitude maps to the format's largest finite
  value: ``scale = float32(amax / FMAX)`` with FMAX = 448 (E4M3) or 57344
  (E5M2); a group whose amax is 0 gets scale 1;
* a scale group is the whole tensor (one scale) or one head (one scale per
  head, over every sequence and valid position of the call); padding
  positions (t >= lens[b]) never enter the abs-max;
* the code is ``FMT_RNE_saturating(float32(x / scale))``: the IEEE fp32
  quotient (correctly rounded) followed by the format's rounding -- two
  roundings, in that order;
* ``dequantise`` returns bf16, the path's compute type: the IEEE fp32 product
  ``decode(code) * scale`` rounded to nearest-even bf16 (a product in fp32,
  then one store rounding).

Layouts: activations are logical ``[B][T][H][D]``; the cache is
``[B][H][L][D]`` and sequence b's position t lands in slot ``dst_start[b] + t``.
"""
import numpy as np

from . import e4m3, e5m2

PER_TENSOR = 0
PER_HEAD = 1

E4M3 = 0
E5M2 = 1
_CODEC = {E4M3: (e4m3, e4m3.E4M3_MAX), E5M2: (e5m2, e5m2.E5M2_MAX)}


def valid_mask(B, T, lens):
    """[B][T] boolean: position t of sequence b is valid when t < lens[b]."""
    lens = np.asarray(lens, dtype=np.int64)
    return np.arange(T)[None, :] < lens[:, None]


def group_amax(x, lens, gran):
    """Abs-max per scale group as float32: shape [1] (per tensor) or [H] (per head).

    x: float32 array [B][T][H][D] holding bf16 values exactly.
    """
    x = np.asarray(x, dtype=np.float32)
    B, T, H, D = x.shape
    mask = valid_mask(B, T, lens)
    a = np.abs(x[mask])                        # [n_valid][H][D]
    if gran == PER_TENSOR:
        return np.array([a.max() if a.size else 0.0], dtype=np.float32)
    if a.shape[0] == 0:
        return np.zeros(H, dtype=np.float32)
    return a.max(axis=(0, 2)).astype(np.float32)


def scales_from_amax(amax, fmt=E4M3):
    """scale = float32(amax / FMAX), or 1 where amax is 0."""
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / np.float32(_CODEC[fmt][1])     # IEEE fp32 division
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quantize(x, scale, gran, fmt=E4M3):
    """float32 [B][T][H][D] -> uint8 codes of the same shape."""
    x = np.asarray(x, dtype=np.float32)
    scale = np.asarray(scale, dtype=np.float32)
    if gran == PER_TENSOR:
        s = scale.reshape(1, 1, 1, 1)
    else:
        s = scale.reshape(1, 1, -1, 1)
    with np.errstate(over="ignore"):           # an overflow to inf saturates below
        y = (x / s).astype(np.float32)        # IEEE fp32 division per element
    return _CODEC[fmt][0].encode(y)


def fill_cache(x, lens, dst_start, cache, scale, gran, fmt=E4M3):
    """Write codes of the valid positions into ``cache`` [B][H][L][D] (in place).

    Slot ``dst_start[b] + t`` of sequence b receives position t < lens[b]
    when that slot lies in [0, L); every other slot keeps its old byte.
    """
    B, T, H, D = x.shape
    L = cache.shape[2]
    codes = quantize(x, scale, gran, fmt)      # [B][T][H][D]
    for b in range(B):
        for t in range(int(lens[b])):
            slot = int(dst_start[b]) + t
            if 0 <= slot < L:
                cache[b, :, slot, :] = codes[b, t]
    return cache


def quantize_kv(x, lens, dst_start, cache, gran, fmt=E4M3):
    """The whole dynamic step: scales from the valid abs-max, then the cache fill.

    Returns the float32 scales ([1] or [H]); ``cache`` is written in place.
    """
    scale = scales_from_amax(group_amax(x, lens, gran), fmt)
    fill_cache(x, lens, dst_start, cache, scale, gran, fmt)
    return scale


def dequantize(codes, scale, gran, head_axis, fmt=E4M3):
    """codes (uint8) -> float64 values ``decode(code) * scale`` (exact in fp64).

    ``head_axis`` names the axis that indexes heads when ``gran`` is per head.
    """
    v = _CODEC[fmt][0].decode(codes)
    scale = np.asarray(scale, dtype=np.float64)
    if gran == PER_TENSOR:
        return v * scale.reshape(())
    shape = [1] * v.ndim
    shape[head_axis] = -1
    return v * scale.reshape(shape)


def bf16_rne_bits(v):
    """float32 values -> uint16 bf16 bit patterns, rounded to nearest even.

    The low 16 bits of the fp32 pattern are dropped after adding half an ulp
    of the kept part, minus one when the kept part is even (so an exact half
    rounds to the even pattern).  Finite inputs; infinities keep their bits.
    NaN inputs become a quiet NaN.
    """
    v = np.asarray(v, dtype=np.float32)
    u = v.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), r).astype(np.uint16)


def dequantise_bf16(codes, scale, gran, head_axis, fmt=E4M3):
    """codes (uint8) -> bf16 bit patterns of ``float32(decode(code) * scale)``.

    decode(code) is exact in fp32, the product is the IEEE fp32 product
    (numpy float32 multiply), and the store to bf16 rounds to nearest even.
    """
    v = _CODEC[fmt][0].decode(codes).astype(np.float32)
    scale = np.asarray(scale, dtype=np.float32)
    if gran == PER_TENSOR:
        s = scale.reshape(())
    else:
        shape = [1] * v.ndim
        shape[head_axis] = -1
        s = scale.reshape(shape)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = (v * s).astype(np.float32)
    return bf16_rne_bits(prod)


def unfill_cache(cache, lens, scale, gran, T, fmt=E4M3):
    """The inverse read of ``fill_cache`` with dst_start = 0: bf16 bits
    [B][T][H][D] with position t < lens[b] set to the dequantised slot t of
    cache [B][H][L][D]; other positions are returned as 0xFFFF (never
    written)."""
    B, H, L, D = cache.shape
    out = np.full((B, T, H, D), 0xFFFF, dtype=np.uint16)
    dq = dequantise_bf16(cache, scale, gran, head_axis=1, fmt=fmt)   # [B][H][L][D]
    for b in range(B):
        n = min(max(int(lens[b]), 0), T, L)
        out[b, :n] = dq[b, :, :n, :].transpose(1, 0, 2)
    return out
