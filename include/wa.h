/*
 * wa.h -- C ABI of the Whisper attention hot path on MI355X (gfx950).
 *
 * Operations, all asynchronous on the caller's HIP stream:
 *
 *   wa_kv_quant_fp8  bf16 -> float8 E4M3 quantization that fills a KV cache
 *                    (wa_kv_quant_fp8_fmt: E4M3 or E5M2; wa_kv_quant_fp8_kv:
 *                    K and V in one call)
 *   wa_kv_dequant_fp8  float8 cache -> bf16, the inverse read
 *   wa_encoder_attn  dense bf16 softmax attention (encoder self-attention,
 *                    or causal decoder prompt prefill), ragged by length
 *                    (wa_encoder_attn_fp8qk: Q and K in E4M3)
 *   wa_decode_attn   one query token per sequence against an E4M3 KV cache
 *                    (decoder self-attention or cross-attention)
 *   wa_decode_attn_append  the same for decoder self-attention, with the
 *                    step's token written into the cache in the same launch
 *   wa_decode_attn_noalloc  wa_decode_attn with no workspace, for callers
 *                    that cannot allocate
 *
 * Sources for what is computed:
 *   - "Blazingly fast whisper transcriptions with Inference Endpoints" (HF
 *     blog), section "Inference Stack": activations are quantized on the fly
 *     and the KV cache is stored as one-byte float8 while computation stays
 *     in bfloat16.
 *   - whisper-blaze 0.1.8 (PyPI page): feature list ("FP8 quantize/dequantize
 *     with per-tensor scaling"; Flash Attention for encoder self-attention
 *     and decoder self/cross-attention) and "Direct Kernel API"
 *     (quantise_e4m3 returns codes and a scale; dequantise_e4m3 takes both;
 *     encoder_self_attn and decoder_cross_attn take no mask, decoder_self_attn
 *     a causal one).
 *   - "Unlocking the power of OpenAI's Whisper", section 3 (encoder
 *     self-attention over the audio frames; decoder self-attention over
 *     previous tokens and cross-attention over the encoded audio).
 *
 * Conventions shared by every call
 *   - Pointers marked "device" point to GPU memory, owned by the caller; the
 *     library allocates nothing and keeps no pointer after a call returns.
 *   - bf16 tensors are passed as uint16_t bit patterns.  head_dim must be 64
 *     (WA_ERR_UNSUPPORTED otherwise); the head_dim axis has stride 1.
 *     Other strides are in elements.  bf16 pointers must be 16-byte aligned
 *     and their b/t/h strides multiples of 8; uint8 cache pointers and
 *     workspaces 16-byte aligned, cache strides multiples of 16
 *     (WA_ERR_UNSUPPORTED otherwise).
 *   - The encoder calls address a row of K or V within 64 rows with a 31-bit
 *     byte offset: a position stride (ks.t, vs.t) of 2^24 elements or more
 *     (2^25 for E4M3 codes) is WA_ERR_UNSUPPORTED.
 *   - Argument checks run on the host before any HIP call and launch nothing
 *     on failure.  The first call on a device checks that it is a gfx950
 *     (WA_ERR_UNSUPPORTED otherwise).  A failed launch returns WA_ERR_HIP.
 *   - Length arrays live on the device, so a decode loop never waits on the
 *     host.  Kernels clamp each length to [0, maximum]; positions at or
 *     beyond a sequence's length are neither read nor written.
 *   - No call synchronises; results are ready when the stream reaches them.
 *     Calls keep no state and may be made from several host threads; two
 *     calls in flight at once must not share a workspace.
 */
#ifndef WA_H
#define WA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WA_OK = 0,
  WA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, bad enum */
  WA_ERR_UNSUPPORTED = 2,        /* head_dim != 64, misalignment, not gfx950 */
  WA_ERR_WORKSPACE_TOO_SMALL = 3,
  WA_ERR_HIP = 4,                /* a HIP runtime call or launch failed */
  WA_ERR_TOO_LARGE = 5           /* more scratch than wa_decode_attn_noalloc holds */
} wa_status;

typedef enum {
  WA_SCALE_PER_TENSOR = 0,       /* one scale for the whole tensor: scale[1] */
  WA_SCALE_PER_HEAD = 1          /* one scale per head: scale[H] */
} wa_scale_gran;

typedef enum {
  WA_FP8_E4M3 = 0,               /* OCP E4M3: bias 7, max 448, NaN only */
  WA_FP8_E5M2 = 1                /* OCP E5M2: bias 15, max 57344, +-inf and NaN */
} wa_fp8_format;

/* Element strides of the batch, position and head axes. */
typedef struct {
  int64_t b, t, h;
} wa_strides;

/*
 * wa_kv_quant_fp8 -- quantize bf16 keys or values into an E4M3 KV cache.
 *
 * What: for every scale group g (the whole tensor, or head h) the
 *   dequantization multiplier is scale[g] = fp32(amax_g / 448), where amax_g
 *   is the largest |x| over the valid positions (t < lens[b]) of that group,
 *   and scale[g] = 1 when amax_g is 0.  Each valid element becomes
 *     code = E4M3(clamp(fp32(x / scale[g]), -448, 448))
 *   with the IEEE fp32 quotient rounded to nearest even, then rounded to
 *   nearest-even OCP E4M3 (max 448, sign kept, so -0 gives 0x80).  So
 *   x ~= decode(code) * scale[g].  The pages name dynamic per-tensor E4M3
 *   scaling (whisper-blaze "Direct Kernel API"; HF blog "Inference Stack");
 *   the scale formula, rounding and per-head groups are the plain reading.
 *
 * x          device, bf16 [B][T_max][H][64] with strides xs.
 * lens       device int32 [B], valid positions per sequence; NULL = T_max.
 * dst_start  device int32 [B]; position t of sequence b goes to cache slot
 *            dst_start[b] + t.  NULL = 0.  Slots outside [0, cache_len) are
 *            skipped; untouched slots keep their bytes.
 * cache      device uint8 [B][H][cache_len][64] with strides cs (t = slot).
 * scale      device float32 [1] or [H] (gran).  compute_scale = 1: written
 *            with the dynamic scales above.  compute_scale = 0: read as given
 *            (a static scale, e.g. appending a decode token to a cache filled
 *            earlier); values beyond 448 * scale saturate.
 * workspace  device scratch of at least wa_kv_quant_fp8_workspace_size()
 *            bytes (only used when compute_scale = 1; may be NULL otherwise).
 *            Its first 256 bytes hold a counter through which the last of
 *            the amax pass's blocks finds itself (that block folds the
 *            scales); it must be zero before
 *            the first call that uses the workspace (a zero-filled
 *            allocation), and every call leaves it zero again, so a
 *            workspace reused call after call needs no further clearing.
 *            The rest needs no initialisation.
 */
wa_status wa_kv_quant_fp8(const uint16_t *x, wa_strides xs, int B, int H, int T_max,
                          int head_dim, const int32_t *lens, const int32_t *dst_start,
                          uint8_t *cache, wa_strides cs, int cache_len, float *scale,
                          wa_scale_gran gran, int compute_scale, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes for one tensor of wa_kv_quant_fp8 (and _fmt) at batch B,
 * H heads and scale granularity gran: a 256-byte counter and the amax pass's
 * partial maxima, at most 32 per sequence and scale group whatever the
 * sequence length.  0 for B <= 0, H <= 0 or an unknown gran. */
size_t wa_kv_quant_fp8_workspace_size(int B, int H, wa_scale_gran gran);

/*
 * wa_kv_quant_fp8_fmt -- wa_kv_quant_fp8 with the float8 format chosen.
 *
 * What: whisper-blaze 0.1.8 (PyPI page, feature list) names both OCP float8
 *   formats, E4M3 and E5M2.  fmt = WA_FP8_E4M3 is exactly wa_kv_quant_fp8.
 *   fmt = WA_FP8_E5M2 replaces 448 by E5M2's largest finite value 57344:
 *     scale[g] = fp32(amax_g / 57344)   (1 when amax_g is 0),
 *     code = E5M2(clamp(fp32(x / scale[g]), -57344, 57344))
 *   rounded to nearest even; codes are never +-inf or NaN.  Arguments,
 *   workspace and errors are those of wa_kv_quant_fp8; a bad fmt is
 *   WA_ERR_INVALID_ARGUMENT.
 */
wa_status wa_kv_quant_fp8_fmt(const uint16_t *x, wa_strides xs, int B, int H, int T_max,
                              int head_dim, const int32_t *lens, const int32_t *dst_start,
                              uint8_t *cache, wa_strides cs, int cache_len, float *scale,
                              wa_scale_gran gran, wa_fp8_format fmt, int compute_scale,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * wa_kv_quant_fp8_kv -- wa_kv_quant_fp8_fmt for a layer's keys and values in
 * one call.
 *
 * What: exactly two wa_kv_quant_fp8_fmt calls, (k -> k_cache, k_scale) and
 *   (v -> v_cache, v_scale), with their own scale groups (the cache fill of
 *   the HF blog's "Inference Stack" stores both K and V in one byte), run as
 *   one launch per kernel instead of two.  K and V share B, H, T_max, lens,
 *   dst_start, the cache layout cs and cache_len; their activation strides
 *   ks and vs may differ.
 *
 * workspace  device scratch of at least 2 * wa_kv_quant_fp8_workspace_size()
 *            bytes when compute_scale = 1: K's part, then V's part starting
 *            wa_kv_quant_fp8_workspace_size() bytes in, each with its own
 *            256-byte counter at its start (zero before first use, left zero
 *            by every call, as for wa_kv_quant_fp8).
 * Errors: those of wa_kv_quant_fp8_fmt; a null v, v_cache or v_scale is
 *   WA_ERR_INVALID_ARGUMENT.
 */
wa_status wa_kv_quant_fp8_kv(const uint16_t *k, wa_strides ks, const uint16_t *v, wa_strides vs,
                             int B, int H, int T_max, int head_dim, const int32_t *lens,
                             const int32_t *dst_start, uint8_t *k_cache, uint8_t *v_cache,
                             wa_strides cs, int cache_len, float *k_scale, float *v_scale,
                             wa_scale_gran gran, wa_fp8_format fmt, int compute_scale,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * wa_kv_dequant_fp8 -- read a float8 KV cache back as bf16.
 *
 * What: the dequantise of whisper-blaze 0.1.8 ("Direct Kernel API":
 *   dequantise_e4m3 takes the codes and the scale quantise_e4m3 returned;
 *   feature list: "FP8 quantize/dequantize with per-tensor scaling").  For
 *   every sequence b, head h and position t < n, n = lens[b] clamped to
 *   [0, min(T_max, cache_len)] (lens NULL: n = min(T_max, cache_len)):
 *     x[b][t][h][:] = bf16(fp32(decode(cache[b][h][t][:]) * scale[g]))
 *   with decode exact in fp32, the IEEE fp32 product, and the store rounded
 *   to nearest even.  Positions t >= n of x are not written.  Codes that
 *   decode to +-inf or NaN (never written by the quantize calls) give +-inf
 *   or a NaN.
 *
 * cache      device uint8 [B][H][cache_len][64] with strides cs (t = slot).
 * scale      device float32 [1] or [H] (gran).
 * lens       device int32 [B] or NULL.
 * x          device bf16 [B][T_max][H][64] with strides xs; must not overlap
 *            the cache.
 * Errors: null pointer, non-positive size or bad enum ->
 *   WA_ERR_INVALID_ARGUMENT; head_dim != 64, B or H above 65535, layout
 *   (alignment, strides) -> WA_ERR_UNSUPPORTED.
 */
wa_status wa_kv_dequant_fp8(const uint8_t *cache, wa_strides cs, int cache_len,
                            const float *scale, wa_scale_gran gran, wa_fp8_format fmt,
                            const int32_t *lens, int B, int H, int T_max, int head_dim,
                            uint16_t *x, wa_strides xs, hipStream_t stream);

/*
 * wa_encoder_attn -- dense softmax attention over bf16 Q/K/V.
 *
 * What: per sequence b, head h and query i < lens[b]:
 *     O[i] = sum_j softmax_j(softmax_scale * Q[i] . K[j]) V[j]
 *   over keys j < lens[b] (causal = 0: encoder self-attention, unmasked in
 *   whisper-blaze "Direct Kernel API") or j <= i (causal = 1: decoder prompt
 *   prefill, masked causally as decoder_self_attn is there).
 *   Accumulation is fp32; O is written as bf16 (round to nearest even).
 *   Rows i >= lens[b] of O are not written.
 *
 * q, k, v    device bf16 [B][T_max][H][64] with strides qs, ks, vs.
 * o          device bf16 [B][T_max][H][64] with strides os; must not alias
 *            q, k or v.
 * lens       device int32 [B]; NULL = T_max for every sequence.
 * softmax_scale  the score multiplier, e.g. 1/sqrt(64) = 0.125.
 */
wa_status wa_encoder_attn(const uint16_t *q, wa_strides qs, const uint16_t *k, wa_strides ks,
                          const uint16_t *v, wa_strides vs, uint16_t *o, wa_strides os, int B,
                          int H, int T_max, int head_dim, const int32_t *lens, int causal,
                          float softmax_scale, hipStream_t stream);

/*
 * wa_cross_attn -- decoder cross-attention for a block of query tokens.
 *
 * What: whisper-blaze's decoder_cross_attn (PyPI page, "Direct Kernel API":
 *   no mask) for several decoder tokens at once, such as a prompt attending to
 *   the encoder's output ("Unlocking the power of OpenAI's Whisper", section
 *   3: the decoder attends over the encoded audio).  Per sequence b and head h,
 *   for query i < q_lens[b]:
 *     O[i] = sum_{j < k_lens[b]} softmax_j(softmax_scale * Q[i] . K[j]) V[j]
 *   with fp32 accumulation, O written as bf16 (round to nearest even).  Rows
 *   i >= q_lens[b] are not written; k_lens[b] = 0 gives zero rows.  With
 *   T_q = T_k and q_lens = k_lens this is wa_encoder_attn with causal = 0.
 *   K and V may be any [B][T_k][H][64] view, e.g. a [B][H][T_k][64] bf16
 *   cache (ks.t = 64, ks.h = T_k * 64); a float8 cache is first expanded with
 *   wa_kv_dequant_fp8.
 *
 * q, o       device bf16 [B][T_q][H][64] with strides qs, os; o must not alias
 *            q, k or v.
 * k, v       device bf16 [B][T_k][H][64] with strides ks, vs.
 * q_lens     device int32 [B] or NULL (= T_q); values clamped to [0, T_q].
 * k_lens     device int32 [B] or NULL (= T_k); values clamped to [0, T_k].
 * Errors: null tensor pointer, non-positive B, H, T_q or T_k, or a
 *   softmax_scale that is not finite and positive -> WA_ERR_INVALID_ARGUMENT;
 *   head_dim != 64, layout (16-byte alignment, strides multiples of 8),
 *   ks.t or vs.t of 2^24 or more -> WA_ERR_UNSUPPORTED.
 */
wa_status wa_cross_attn(const uint16_t *q, wa_strides qs, const uint16_t *k, wa_strides ks,
                        const uint16_t *v, wa_strides vs, uint16_t *o, wa_strides os, int B, int H,
                        int T_q, int T_k, int head_dim, const int32_t *q_lens,
                        const int32_t *k_lens, float softmax_scale, hipStream_t stream);

/*
 * wa_encoder_attn_fp8qk -- wa_encoder_attn with Q and K given in float8 E4M3.
 *
 * What: whisper-blaze 0.1.8's "aggressive_fp8" preset (PyPI page, "Precision
 *   Presets": FP8 everywhere) read for attention as Q and K stored as E4M3
 *   codes with the quantize step's scales (V and the output stay bf16):
 *     O = wa_encoder_attn(Q^, K^, V),  Q^ = decode(Qc) * q_scale[g],
 *                                      K^ = decode(Kc) * k_scale[g]
 *   with g = 0 (WA_SCALE_PER_TENSOR) or the head (WA_SCALE_PER_HEAD).  The
 *   scores are taken on the fp8 matrix cores (v_mfma_f32_32x32x64_f8f6f4,
 *   fp32 result; its internal sums round at about 1e-4 of the sum of the
 *   products' magnitudes), then scaled by softmax_scale * q_scale * k_scale.
 *   Masks, lengths and rows not written are those of wa_encoder_attn.  The
 *   codes are what wa_kv_quant_fp8 writes when given [B][T][H][64] strides.
 *
 * q, k       device uint8 [B][T_max][H][64] with strides qs, ks (in bytes:
 *            16-byte aligned, strides multiples of 16).
 * q_scale, k_scale  device float32 [1] or [H] (gran).
 * v, o, lens, causal, softmax_scale, errors: as wa_encoder_attn; a null
 *            scale is WA_ERR_INVALID_ARGUMENT.
 */
wa_status wa_encoder_attn_fp8qk(const uint8_t *q, wa_strides qs, const float *q_scale,
                                const uint8_t *k, wa_strides ks, const float *k_scale,
                                wa_scale_gran gran, const uint16_t *v, wa_strides vs, uint16_t *o,
                                wa_strides os, int B, int H, int T_max, int head_dim,
                                const int32_t *lens, int causal, float softmax_scale,
                                hipStream_t stream);

/*
 * wa_decode_attn -- one query token per sequence against an E4M3 KV cache.
 *
 * What: per sequence b and head h, with n = lens[b] cached slots,
 *     K^_j = decode(Kc[b,h,j]) * k_scale[g],  V^_j likewise (g = 0 or h),
 *     o = sum_{j<n} softmax_j(softmax_scale * q . K^_j) V^_j
 *   computed in fp32 from the bf16 query, written as bf16.  The query sits at
 *   the last cached position, so the causal decoder self-attention of
 *   whisper-blaze's decoder_self_attn sees every slot j < n (its own K/V
 *   already appended at slot n - 1); cross-attention (decoder_cross_attn, no
 *   mask) passes n = 1500 for every sequence.  n = 0 gives a zero row.  The
 *   keys are split into chunks evaluated in parallel and merged with the
 *   softmax rescaling identity.
 *
 * q          device bf16 [B][H][64]; qs.b and qs.h used (qs.t ignored).
 * k_cache, v_cache  device uint8 [B][H][cache_len][64], both with strides cs.
 * k_scale, v_scale  device float32 [1] or [H] (gran).
 * lens       device int32 [B] (required).
 * o          device bf16 [B][H][64]; os.b and os.h used.
 * workspace  device scratch of at least wa_decode_attn_workspace_size() bytes
 *            (0 when the keys are not split; NULL is then allowed).  It
 *            begins with one counter per (b, h), through which the last of a
 *            pair's chunk blocks finds itself and merges the chunks, so the
 *            workspace must be zero before the first call that uses it (a
 *            zero-filled allocation); every call leaves the counters zero
 *            again, so a workspace reused call after call needs no further
 *            clearing.
 */
wa_status wa_decode_attn(const uint16_t *q, wa_strides qs, const uint8_t *k_cache,
                         const uint8_t *v_cache, wa_strides cs, int cache_len,
                         const float *k_scale, const float *v_scale, wa_scale_gran gran,
                         const int32_t *lens, int B, int H, int head_dim, float softmax_scale,
                         uint16_t *o, wa_strides os, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

size_t wa_decode_attn_workspace_size(int B, int H, int cache_len);

/*
 * wa_decode_attn_append -- one decoder self-attention step that also appends
 * the step's token to the cache, in one launch.
 *
 * What: the decode-step append of the HF blog's float8 KV cache ("Blazingly
 *   fast whisper transcriptions with Inference Endpoints", section
 *   "Inference Stack": each new token's keys and values are stored in one
 *   byte) followed by whisper-blaze's decoder_self_attn for that token
 *   (whisper-blaze 0.1.8, "Direct Kernel API").  Per sequence b and head h,
 *   with n = lens[b] clamped to [0, cache_len] and n counting the new token:
 *     Kc[b,h,n-1] = E4M3(k_new[b,h] / k_scale[g]),  Vc[b,h,n-1] likewise,
 *   exactly the codes wa_kv_quant_fp8 with compute_scale = 0 and
 *   dst_start = n - 1 writes; then o as in wa_decode_attn over the n slots.
 *   Slots other than n - 1 are read, never written.  n = 0 writes nothing
 *   and gives a zero row.
 *
 * k_new, v_new  device bf16 [B][H][64], strides ns (ns.b, ns.h; ns.t ignored).
 * k_cache, v_cache  device uint8 [B][H][cache_len][64], written at slot n-1.
 * Other arguments, the workspace (wa_decode_attn_workspace_size) and the
 * errors are those of wa_decode_attn.
 */
wa_status wa_decode_attn_append(const uint16_t *q, wa_strides qs, const uint16_t *k_new,
                                const uint16_t *v_new, wa_strides ns, uint8_t *k_cache,
                                uint8_t *v_cache, wa_strides cs, int cache_len,
                                const float *k_scale, const float *v_scale, wa_scale_gran gran,
                                const int32_t *lens, int B, int H, int head_dim,
                                float softmax_scale, uint16_t *o, wa_strides os, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * wa_decode_attn_noalloc -- wa_decode_attn for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  It takes no workspace and allocates
 * nothing; inputs, outputs and errors are those of wa_decode_attn (same
 * kernels, bit-identical results).
 *
 * The split-key counters and partials go to a static device array of
 * WA_DECODE_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds
 * until the process ends (zero when the library loads; every call leaves
 * its counters zero).  A call whose scratch (the bytes
 * wa_decode_attn_workspace_size reports) exceeds it returns
 * WA_ERR_TOO_LARGE and launches nothing; with the current planner no call
 * needs more than about 455 KB.  Every call on a GPU shares that GPU's array: two calls in
 * flight at once on one GPU (on two streams, or from two host threads) race
 * and must not overlap.
 */
#define WA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)512 * 1024)

wa_status wa_decode_attn_noalloc(const uint16_t *q, wa_strides qs, const uint8_t *k_cache,
                                 const uint8_t *v_cache, wa_strides cs, int cache_len,
                                 const float *k_scale, const float *v_scale, wa_scale_gran gran,
                                 const int32_t *lens, int B, int H, int head_dim,
                                 float softmax_scale, uint16_t *o, wa_strides os,
                                 hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *wa_status_string(wa_status s);

#ifdef __cplusplus
}
#endif

#endif /* WA_H */
