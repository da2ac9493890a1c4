"""Python binding of libwa.so, the C-ABI library of the Whisper attention hot path.

Argument marshalling only: every step runs in the HIP kernels behind
``include/wa.h``.  PyTorch provides device memory and the current stream.
The functions keep the C names:

* ``wa_kv_quant_fp8``  bf16 -> E4M3 KV-cache fill with dynamic or static scales
  (``wa_kv_quant_fp8_fmt``: E4M3 or E5M2)
* ``wa_kv_dequant_fp8``  float8 cache -> bf16
* ``wa_encoder_attn``  dense bf16 attention (encoder, or causal prompt prefill)
  (``wa_encoder_attn_fp8qk``: E4M3 Q and K)
* ``wa_cross_attn``    decoder cross-attention for several query tokens (query
  and key lengths differ)
* ``wa_decode_attn``   one query token per sequence against an E4M3 cache
  (``wa_decode_attn_noalloc``: no workspace, for callers that cannot allocate)

The library must have been built (``python whisper_attention_amd/build.py``);
importing fails loudly when it is missing -- there is no fallback.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwa.so")

WA_OK = 0
WA_ERR_INVALID_ARGUMENT = 1
WA_ERR_UNSUPPORTED = 2
WA_ERR_WORKSPACE_TOO_SMALL = 3
WA_ERR_HIP = 4
WA_ERR_TOO_LARGE = 5

WA_DECODE_NOALLOC_SCRATCH_BYTES = 512 * 1024

WA_SCALE_PER_TENSOR = 0
WA_SCALE_PER_HEAD = 1

WA_FP8_E4M3 = 0
WA_FP8_E5M2 = 1

HEAD_DIM = 64


class Strides(ctypes.Structure):
    """wa_strides: element strides of the batch, position and head axes."""
    _fields_ = [("b", ctypes.c_int64), ("t", ctypes.c_int64), ("h", ctypes.c_int64)]


class WaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python whisper_attention_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S, F, Z = ctypes.c_void_p, ctypes.c_int, Strides, ctypes.c_float, ctypes.c_size_t
    lib.wa_kv_quant_fp8.argtypes = [P, S, I, I, I, I, P, P, P, S, I, P, I, I, P, Z, P]
    lib.wa_kv_quant_fp8.restype = I
    lib.wa_kv_quant_fp8_fmt.argtypes = [P, S, I, I, I, I, P, P, P, S, I, P, I, I, I, P, Z, P]
    lib.wa_kv_quant_fp8_fmt.restype = I
    lib.wa_kv_quant_fp8_kv.argtypes = [P, S, P, S, I, I, I, I, P, P, P, P, S, I, P, P, I, I, I, P, Z, P]
    lib.wa_kv_quant_fp8_kv.restype = I
    lib.wa_kv_dequant_fp8.argtypes = [P, S, I, P, I, I, P, I, I, I, I, P, S, P]
    lib.wa_kv_dequant_fp8.restype = I
    lib.wa_kv_quant_fp8_workspace_size.argtypes = [I, I, I]
    lib.wa_kv_quant_fp8_workspace_size.restype = Z
    lib.wa_encoder_attn.argtypes = [P, S, P, S, P, S, P, S, I, I, I, I, P, I, F, P]
    lib.wa_encoder_attn.restype = I
    lib.wa_encoder_attn_fp8qk.argtypes = [P, S, P, P, S, P, I, P, S, P, S, I, I, I, I, P, I, F, P]
    lib.wa_encoder_attn_fp8qk.restype = I
    lib.wa_cross_attn.argtypes = [P, S, P, S, P, S, P, S, I, I, I, I, I, P, P, F, P]
    lib.wa_cross_attn.restype = I
    lib.wa_decode_attn.argtypes = [P, S, P, P, S, I, P, P, I, P, I, I, I, F, P, S, P, Z, P]
    lib.wa_decode_attn.restype = I
    lib.wa_decode_attn_append.argtypes = [P, S, P, P, S, P, P, S, I, P, P, I, P, I, I, I, F, P, S, P, Z, P]
    lib.wa_decode_attn_append.restype = I
    lib.wa_decode_attn_noalloc.argtypes = [P, S, P, P, S, I, P, P, I, P, I, I, I, F, P, S, P]
    lib.wa_decode_attn_noalloc.restype = I
    lib.wa_decode_attn_workspace_size.argtypes = [I, I, I]
    lib.wa_decode_attn_workspace_size.restype = Z
    lib.wa_status_string.argtypes = [I]
    lib.wa_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()

EXPORTED = ("wa_kv_quant_fp8", "wa_kv_quant_fp8_fmt", "wa_kv_quant_fp8_kv", "wa_kv_dequant_fp8",
            "wa_kv_quant_fp8_workspace_size", "wa_encoder_attn", "wa_encoder_attn_fp8qk",
            "wa_cross_attn", "wa_decode_attn", "wa_decode_attn_append", "wa_decode_attn_noalloc",
            "wa_decode_attn_workspace_size", "wa_status_string")


def wa_status_string(status):
    return lib.wa_status_string(int(status)).decode()


def _check(status):
    if status != WA_OK:
        raise WaError(status, wa_status_string(status))


def _gran(g):
    if g in ("tensor", WA_SCALE_PER_TENSOR):
        return WA_SCALE_PER_TENSOR
    if g in ("head", WA_SCALE_PER_HEAD):
        return WA_SCALE_PER_HEAD
    raise ValueError(f"scale granularity {g!r}")


def _fmt(f):
    if f in ("e4m3", WA_FP8_E4M3):
        return WA_FP8_E4M3
    if f in ("e5m2", WA_FP8_E5M2):
        return WA_FP8_E5M2
    raise ValueError(f"float8 format {f!r}")


def _ptr(t):
    """Device pointer of a GPU tensor (None passes through).  The kernels
    dereference every pointer on the device, so a host tensor is refused."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor (the library reads every buffer on the device)")
    return ctypes.c_void_p(t.data_ptr())


def _vec(t, dtype, n, what):
    """A contiguous device vector of at least n elements (lengths, slots, scales)."""
    if t is None:
        return None
    if t.dtype != dtype or t.dim() != 1 or t.numel() < n or not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous {dtype} vector of at least {n} elements, "
                         f"got {t.dtype} {tuple(t.shape)}")
    return _ptr(t)


def _stream(t, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _act_strides(t):
    """[B][T][H][D] tensor -> wa_strides(b, t, h)."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B][T][H][64] tensor with a contiguous last axis")
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def _cache_strides(t):
    """[B][H][L][D] cache -> wa_strides(b, t=slot, h)."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B][H][L][64] cache with a contiguous last axis")
    return Strides(t.stride(0), t.stride(2), t.stride(1))


def _tok_strides(t):
    """[B][H][D] token tensor -> wa_strides(b, 0, h)."""
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError("expected a [B][H][64] tensor with a contiguous last axis")
    return Strides(t.stride(0), 0, t.stride(1))


def _bits(t, dtype):
    if t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t


def _shape(t, want, what):
    """Refuse a tensor whose shape differs from ``want`` (None entries are
    free): the kernels take every size from one tensor, so a mismatched one
    would be read or written out of its bounds."""
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and g != w for g, w in zip(got, want)):
        shown = "][".join("*" if w is None else str(w) for w in want)
        raise ValueError(f"{what}: expected shape [{shown}], got {list(got)}")


def _same_device(ref, *ts):
    for t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"every tensor must be on {ref.device}; got one on {t.device}")


def wa_kv_quant_fp8_workspace_size(B, H, gran):
    return int(lib.wa_kv_quant_fp8_workspace_size(B, H, _gran(gran)))


def wa_decode_attn_workspace_size(B, H, cache_len):
    return int(lib.wa_decode_attn_workspace_size(B, H, cache_len))


def wa_kv_quant_fp8(x, cache, scale, gran, lens=None, dst_start=None, compute_scale=True,
                    workspace=None, stream=None):
    """Quantize bf16 ``x`` [B][T][H][64] into the uint8 E4M3 ``cache`` [B][H][L][64].

    ``scale`` (float32, [1] or [H]) is written when ``compute_scale`` and read
    otherwise.  ``lens``/``dst_start`` are int32 device tensors [B] or None.
    A ``workspace`` passed in must have been zero-filled before its first use
    (every call leaves its counter at zero).
    """
    return wa_kv_quant_fp8_fmt(x, cache, scale, gran, "e4m3", lens, dst_start, compute_scale,
                               workspace, stream)


def wa_kv_quant_fp8_fmt(x, cache, scale, gran, fmt, lens=None, dst_start=None, compute_scale=True,
                        workspace=None, stream=None):
    """``wa_kv_quant_fp8`` with the format chosen: ``fmt`` is "e4m3" or "e5m2"."""
    _bits(x, torch.bfloat16)
    _bits(cache, torch.uint8)
    _bits(scale, torch.float32)
    B, T, H, D = x.shape
    _shape(cache, (B, H, None, D), "cache")
    _same_device(x, cache, scale, lens, dst_start, workspace)
    g = _gran(gran)
    if workspace is None and compute_scale:
        n = wa_kv_quant_fp8_workspace_size(B, H, g)
        # zero-filled: the workspace begins with the scale fold's counter
        workspace = torch.zeros(max(n, 16), dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ng = 1 if g == WA_SCALE_PER_TENSOR else H
    _check(lib.wa_kv_quant_fp8_fmt(_ptr(x), _act_strides(x), B, H, T, D, _vec(lens, torch.int32, B, "lens"),
                                   _vec(dst_start, torch.int32, B, "dst_start"), _ptr(cache),
                                   _cache_strides(cache), cache.shape[2],
                                   _vec(scale, torch.float32, ng, "scale"), g, _fmt(fmt),
                                   int(bool(compute_scale)), _ptr(workspace), ws_bytes,
                                   _stream(x, stream)))
    return scale


def wa_kv_quant_fp8_kv(k, v, k_cache, v_cache, k_scale, v_scale, gran, fmt="e4m3", lens=None,
                       dst_start=None, compute_scale=True, workspace=None, stream=None):
    """K and V [B][T][H][64] bf16 into their uint8 caches [B][H][L][64] (same
    layout) and scales, in one call; see ``wa_kv_quant_fp8_fmt``."""
    for t in (k, v):
        _bits(t, torch.bfloat16)
    for t in (k_cache, v_cache):
        _bits(t, torch.uint8)
    for t in (k_scale, v_scale):
        _bits(t, torch.float32)
    if k.shape != v.shape or k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k/v and their caches must share shapes, and the caches their strides")
    B, T, H, D = k.shape
    _shape(k_cache, (B, H, None, D), "k_cache")
    _same_device(k, v, k_cache, v_cache, k_scale, v_scale, lens, dst_start, workspace)
    g = _gran(gran)
    if workspace is None and compute_scale:
        n = 2 * wa_kv_quant_fp8_workspace_size(B, H, g)
        # zero-filled: each half begins with the scale fold's counter
        workspace = torch.zeros(max(n, 16), dtype=torch.uint8, device=k.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ng = 1 if g == WA_SCALE_PER_TENSOR else H
    _check(lib.wa_kv_quant_fp8_kv(_ptr(k), _act_strides(k), _ptr(v), _act_strides(v), B, H, T, D,
                                  _vec(lens, torch.int32, B, "lens"), _vec(dst_start, torch.int32, B, "dst_start"),
                                  _ptr(k_cache), _ptr(v_cache), _cache_strides(k_cache), k_cache.shape[2],
                                  _vec(k_scale, torch.float32, ng, "k_scale"),
                                  _vec(v_scale, torch.float32, ng, "v_scale"),
                                  g, _fmt(fmt), int(bool(compute_scale)), _ptr(workspace), ws_bytes,
                                  _stream(k, stream)))
    return k_scale, v_scale


def wa_kv_dequant_fp8(cache, scale, gran, fmt, out=None, T_max=None, lens=None, stream=None):
    """Read the uint8 ``cache`` [B][H][L][64] back as bf16 ``out`` [B][T][H][64]
    (T = ``T_max``, default L): positions t < lens[b] (all when ``lens`` is
    None) are written, the others are left as they are."""
    _bits(cache, torch.uint8)
    _bits(scale, torch.float32)
    B, H, L, D = cache.shape
    if out is None:
        out = torch.empty((B, L if T_max is None else T_max, H, D), dtype=torch.bfloat16,
                          device=cache.device)
    _bits(out, torch.bfloat16)
    if out.dim() != 4 or (out.shape[0], out.shape[2], out.shape[3]) != (B, H, D):
        raise ValueError(f"out must be [B={B}][T][H={H}][{D}], got {tuple(out.shape)}")
    _same_device(cache, scale, out, lens)
    T = out.shape[1]
    g = _gran(gran)
    ng = 1 if g == WA_SCALE_PER_TENSOR else H
    _check(lib.wa_kv_dequant_fp8(_ptr(cache), _cache_strides(cache), L, _vec(scale, torch.float32, ng, "scale"),
                                 g, _fmt(fmt), _vec(lens, torch.int32, B, "lens"), B, H, T, D, _ptr(out),
                                 _act_strides(out),
                                 _stream(cache, stream)))
    return out


def wa_encoder_attn(q, k, v, out=None, lens=None, causal=False, softmax_scale=0.125, stream=None):
    """Dense bf16 attention over [B][T][H][64] tensors; returns ``out``."""
    for t in (q, k, v):
        _bits(t, torch.bfloat16)
    B, T, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _bits(out, torch.bfloat16)
    for t, name in ((k, "k"), (v, "v"), (out, "out")):
        _shape(t, (B, T, H, D), name)
    _same_device(q, k, v, out, lens)
    _check(lib.wa_encoder_attn(_ptr(q), _act_strides(q), _ptr(k), _act_strides(k), _ptr(v),
                               _act_strides(v), _ptr(out), _act_strides(out), B, H, T, D,
                               _vec(lens, torch.int32, B, "lens"), int(bool(causal)), float(softmax_scale),
                               _stream(q, stream)))
    return out


def wa_encoder_attn_fp8qk(q, q_scale, k, k_scale, gran, v, out=None, lens=None, causal=False,
                          softmax_scale=0.125, stream=None):
    """Dense attention with E4M3 Q and K (uint8 [B][T][H][64] codes, float32
    scales [1] or [H]) and bf16 V [B][T][H][64]; returns ``out`` (bf16)."""
    _bits(q, torch.uint8)
    _bits(k, torch.uint8)
    _bits(v, torch.bfloat16)
    _bits(q_scale, torch.float32)
    _bits(k_scale, torch.float32)
    B, T, H, D = v.shape
    if q.shape != v.shape or k.shape != v.shape:
        raise ValueError("q, k and v must share the [B][T][H][64] shape")
    if out is None:
        out = torch.empty_like(v)
    _bits(out, torch.bfloat16)
    _shape(out, (B, T, H, D), "out")
    _same_device(v, q, k, q_scale, k_scale, out, lens)
    g = _gran(gran)
    ng = 1 if g == WA_SCALE_PER_TENSOR else H
    _check(lib.wa_encoder_attn_fp8qk(_ptr(q), _act_strides(q), _vec(q_scale, torch.float32, ng, "q_scale"),
                                     _ptr(k), _act_strides(k), _vec(k_scale, torch.float32, ng, "k_scale"),
                                     g, _ptr(v), _act_strides(v), _ptr(out), _act_strides(out), B, H, T, D,
                                     _vec(lens, torch.int32, B, "lens"), int(bool(causal)),
                                     float(softmax_scale), _stream(v, stream)))
    return out


def wa_cross_attn(q, k, v, out=None, q_lens=None, k_lens=None, softmax_scale=0.125, stream=None):
    """Cross-attention of bf16 queries [B][Tq][H][64] over bf16 keys and
    values [B][Tk][H][64] (any strided views); returns ``out``."""
    for t in (q, k, v):
        _bits(t, torch.bfloat16)
    B, Tq, H, D = q.shape
    Tk = k.shape[1]
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != q.shape[2:]:
        raise ValueError("k and v must be [B][Tk][H][64] with q's B, H and head size")
    if out is None:
        out = torch.empty_like(q)
    _bits(out, torch.bfloat16)
    _shape(out, (B, Tq, H, D), "out")
    _same_device(q, k, v, out, q_lens, k_lens)
    _check(lib.wa_cross_attn(_ptr(q), _act_strides(q), _ptr(k), _act_strides(k), _ptr(v),
                             _act_strides(v), _ptr(out), _act_strides(out), B, H, Tq, Tk, D,
                             _vec(q_lens, torch.int32, B, "q_lens"), _vec(k_lens, torch.int32, B, "k_lens"),
                             float(softmax_scale), _stream(q, stream)))
    return out


def wa_decode_attn(q, k_cache, v_cache, k_scale, v_scale, lens, gran, softmax_scale=0.125,
                   out=None, workspace=None, stream=None):
    """One query token per (b, h): q [B][H][64] bf16 against uint8 caches [B][H][L][64]."""
    _bits(q, torch.bfloat16)
    _bits(k_cache, torch.uint8)
    _bits(v_cache, torch.uint8)
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    B, H, D = q.shape
    _shape(k_cache, (B, H, None, D), "k_cache")
    L = k_cache.shape[2]
    if out is None:
        out = torch.empty_like(q)
    _bits(out, torch.bfloat16)
    _shape(out, (B, H, D), "out")
    if workspace is None:
        n = wa_decode_attn_workspace_size(B, H, L)
        # zero-filled: a split-key call's workspace begins with its counters
        workspace = torch.zeros(max(n, 16), dtype=torch.uint8, device=q.device)
    _same_device(q, k_cache, v_cache, k_scale, v_scale, lens, out, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    g = _gran(gran)
    ng = 1 if g == WA_SCALE_PER_TENSOR else H
    _check(lib.wa_decode_attn(_ptr(q), _tok_strides(q), _ptr(k_cache), _ptr(v_cache),
                              _cache_strides(k_cache), L, _vec(k_scale, torch.float32, ng, "k_scale"),
                              _vec(v_scale, torch.float32, ng, "v_scale"), g,
                              _vec(lens, torch.int32, B, "lens"), B, H, D, float(softmax_scale), _ptr(out),
                              _tok_strides(out), _ptr(workspace), ws_bytes, _stream(q, stream)))
    return out


def wa_decode_attn_append(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, lens, gran,
                          softmax_scale=0.125, out=None, workspace=None, stream=None):
    """Append the step's token (k_new, v_new: [B][H][64] bf16) to the uint8
    caches at slot lens[b] - 1 with the stored scales, then attend q to the
    lens[b] slots, in one launch."""
    for t in (q, k_new, v_new):
        _bits(t, torch.bfloat16)
    _bits(k_cache, torch.uint8)
    _bits(v_cache, torch.uint8)
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if k_new.stride() != v_new.stride() or k_new.shape != q.shape or v_new.shape != q.shape:
        raise ValueError("k_new and v_new must have q's shape and share strides")
    B, H, D = q.shape
    _shape(k_cache, (B, H, None, D), "k_cache")
    L = k_cache.shape[2]
    if out is None:
        out = torch.empty_like(q)
    _bits(out, torch.bfloat16)
    _shape(out, (B, H, D), "out")
    if workspace is None:
        n = wa_decode_attn_workspace_size(B, H, L)
        # zero-filled: a split-key call's workspace begins with its counters
        workspace = torch.zeros(max(n, 16), dtype=torch.uint8, device=q.device)
    _same_device(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, lens, out, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    g = _gran(gran)
    ng = 1 if g == WA_SCALE_PER_TENSOR else H
    _check(lib.wa_decode_attn_append(_ptr(q), _tok_strides(q), _ptr(k_new), _ptr(v_new),
                                     _tok_strides(k_new), _ptr(k_cache), _ptr(v_cache),
                                     _cache_strides(k_cache), L, _vec(k_scale, torch.float32, ng, "k_scale"),
                                     _vec(v_scale, torch.float32, ng, "v_scale"), g,
                                     _vec(lens, torch.int32, B, "lens"), B, H, D, float(softmax_scale),
                                     _ptr(out), _tok_strides(out), _ptr(workspace), ws_bytes,
                                     _stream(q, stream)))
    return out


def wa_decode_attn_noalloc(q, k_cache, v_cache, k_scale, v_scale, lens, gran, out, softmax_scale=0.125,
                           stream=None):
    """``wa_decode_attn`` without a workspace: the library keeps the split-key
    partials in a static device array (WA_DECODE_NOALLOC_SCRATCH_BYTES per
    GPU), so neither the call nor this wrapper allocates; ``out`` [B][H][64]
    bf16 is required.  Calls on one GPU must not overlap in time."""
    _bits(q, torch.bfloat16)
    _bits(k_cache, torch.uint8)
    _bits(v_cache, torch.uint8)
    _bits(out, torch.bfloat16)
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    B, H, D = q.shape
    _shape(k_cache, (B, H, None, D), "k_cache")
    _shape(out, (B, H, D), "out")
    _same_device(q, k_cache, v_cache, k_scale, v_scale, lens, out)
    L = k_cache.shape[2]
    g = _gran(gran)
    ng = 1 if g == WA_SCALE_PER_TENSOR else H
    _check(lib.wa_decode_attn_noalloc(_ptr(q), _tok_strides(q), _ptr(k_cache), _ptr(v_cache),
                                      _cache_strides(k_cache), L, _vec(k_scale, torch.float32, ng, "k_scale"),
                                      _vec(v_scale, torch.float32, ng, "v_scale"), g,
                                      _vec(lens, torch.int32, B, "lens"), B, H, D, float(softmax_scale),
                                      _ptr(out), _tok_strides(out), _stream(q, stream)))
    return out
