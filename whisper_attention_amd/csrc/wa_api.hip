// Host entry points of the C ABI declared in include/wa.h: argument checks
// (before any HIP call), the gfx950 check, plan/workspace sizing and the
// kernel launches.  No device memory is allocated here.
#include <cmath>
#include <cstring>
#include <mutex>

#include "wa_internal.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool bf16_layout_ok(const void *p, wa_strides s) {
  return aligned16(p) && s.b % 8 == 0 && s.t % 8 == 0 && s.h % 8 == 0;
}
bool u8_layout_ok(const void *p, wa_strides s) {
  return aligned16(p) && s.b % 16 == 0 && s.t % 16 == 0 && s.h % 16 == 0;
}

// The first call on each device checks that it is a gfx950.
constexpr int kMaxDevices = 64;
std::once_flag g_arch_once[kMaxDevices];
int g_arch_ok[kMaxDevices];

}  // namespace

wa_status wa::check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return WA_ERR_HIP;
  if (dev >= kMaxDevices) return WA_ERR_UNSUPPORTED;
  std::call_once(g_arch_once[dev], [dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      g_arch_ok[dev] = -1;
      return;
    }
    g_arch_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  });
  if (g_arch_ok[dev] < 0) return WA_ERR_HIP;
  return g_arch_ok[dev] ? WA_OK : WA_ERR_UNSUPPORTED;
}

namespace {

using wa::check_device;

wa_status from_hip(hipError_t e) { return e == hipSuccess ? WA_OK : WA_ERR_HIP; }

// A row within 64 rows at a position stride of t elements of elem_bytes (2 or
// 1), addressed with a 31-bit byte offset: t below 2^24 (bf16) or 2^25 (E4M3).
bool tile_rows_fit(int64_t t, int elem_bytes) {
  return t >= 0 && t < (int64_t(1) << (elem_bytes == 2 ? 24 : 25));
}

}  // namespace

extern "C" {

const char *wa_status_string(wa_status s) {
  switch (s) {
    case WA_OK: return "WA_OK";
    case WA_ERR_INVALID_ARGUMENT: return "WA_ERR_INVALID_ARGUMENT: null pointer, non-positive size or bad enum";
    case WA_ERR_UNSUPPORTED: return "WA_ERR_UNSUPPORTED: head_dim != 64, misaligned pointer/stride, or device is not gfx950";
    case WA_ERR_WORKSPACE_TOO_SMALL: return "WA_ERR_WORKSPACE_TOO_SMALL";
    case WA_ERR_HIP: return "WA_ERR_HIP: a HIP runtime call or kernel launch failed";
    case WA_ERR_TOO_LARGE: return "WA_ERR_TOO_LARGE: the call needs more scratch than the no-allocation entry point's static buffer holds";
  }
  return "unknown wa_status";
}

size_t wa_kv_quant_fp8_workspace_size(int B, int H, wa_scale_gran gran) {
  if (B <= 0 || H <= 0) return 0;
  if (gran != WA_SCALE_PER_TENSOR && gran != WA_SCALE_PER_HEAD) return 0;
  return wa::quant_workspace_bytes(B, gran == WA_SCALE_PER_HEAD ? H : 1);
}

}  // extern "C"

namespace {

// One tensor (v == nullptr) or a K/V pair sharing shape, lengths, slots and
// cache layout.
wa_status quant_common(const uint16_t *k, wa_strides ks, const uint16_t *v, wa_strides vs, int B,
                       int H, int T_max, int head_dim, const int32_t *lens,
                       const int32_t *dst_start, uint8_t *k_cache, uint8_t *v_cache,
                       wa_strides cs, int cache_len, float *k_scale, float *v_scale,
                       wa_scale_gran gran, wa_fp8_format fmt, int compute_scale, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  const int n = v ? 2 : 1;
  if (!k || !k_cache || !k_scale) return WA_ERR_INVALID_ARGUMENT;
  if (n == 2 && (!v_cache || !v_scale)) return WA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || T_max <= 0 || cache_len <= 0) return WA_ERR_INVALID_ARGUMENT;
  if (gran != WA_SCALE_PER_TENSOR && gran != WA_SCALE_PER_HEAD) return WA_ERR_INVALID_ARGUMENT;
  if (fmt != WA_FP8_E4M3 && fmt != WA_FP8_E5M2) return WA_ERR_INVALID_ARGUMENT;
  if (compute_scale != 0 && compute_scale != 1) return WA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64) return WA_ERR_UNSUPPORTED;
  if (H > 8192 || T_max > 65535 * 8) return WA_ERR_UNSUPPORTED;
  if (!bf16_layout_ok(k, ks) || !u8_layout_ok(k_cache, cs)) return WA_ERR_UNSUPPORTED;
  if (n == 2 && (!bf16_layout_ok(v, vs) || !u8_layout_ok(v_cache, cs))) return WA_ERR_UNSUPPORTED;
  const wa::QuantPlan plan = wa::quant_plan(B, H, T_max, gran);
  if (compute_scale) {
    if (!workspace) return WA_ERR_INVALID_ARGUMENT;
    if (!aligned16(workspace)) return WA_ERR_UNSUPPORTED;
    if (workspace_bytes < n * wa::quant_workspace_bytes(B, plan.groups)) return WA_ERR_WORKSPACE_TOO_SMALL;
  }
  wa_status st = check_device();
  if (st != WA_OK) return st;
  wa::QuantTensors qt = {{k, v}, {ks, vs}, {k_cache, v_cache}, {k_scale, v_scale}};
  return from_hip(wa::launch_kv_quant(qt, n, B, H, T_max, lens, dst_start, cs, cache_len,
                                      gran == WA_SCALE_PER_HEAD, compute_scale,
                                      fmt == WA_FP8_E4M3 ? wa::Fp8::E4M3 : wa::Fp8::E5M2,
                                      static_cast<uint32_t *>(workspace), plan, stream));
}

}  // namespace

extern "C" {

wa_status wa_kv_quant_fp8_fmt(const uint16_t *x, wa_strides xs, int B, int H, int T_max,
                              int head_dim, const int32_t *lens, const int32_t *dst_start,
                              uint8_t *cache, wa_strides cs, int cache_len, float *scale,
                              wa_scale_gran gran, wa_fp8_format fmt, int compute_scale,
                              void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return quant_common(x, xs, nullptr, wa_strides{0, 0, 0}, B, H, T_max, head_dim, lens, dst_start,
                      cache, nullptr, cs, cache_len, scale, nullptr, gran, fmt, compute_scale,
                      workspace, workspace_bytes, stream);
}

wa_status wa_kv_quant_fp8_kv(const uint16_t *k, wa_strides ks, const uint16_t *v, wa_strides vs,
                             int B, int H, int T_max, int head_dim, const int32_t *lens,
                             const int32_t *dst_start, uint8_t *k_cache, uint8_t *v_cache,
                             wa_strides cs, int cache_len, float *k_scale, float *v_scale,
                             wa_scale_gran gran, wa_fp8_format fmt, int compute_scale,
                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!v) return WA_ERR_INVALID_ARGUMENT;
  return quant_common(k, ks, v, vs, B, H, T_max, head_dim, lens, dst_start, k_cache, v_cache, cs,
                      cache_len, k_scale, v_scale, gran, fmt, compute_scale, workspace,
                      workspace_bytes, stream);
}

wa_status wa_kv_quant_fp8(const uint16_t *x, wa_strides xs, int B, int H, int T_max,
                          int head_dim, const int32_t *lens, const int32_t *dst_start,
                          uint8_t *cache, wa_strides cs, int cache_len, float *scale,
                          wa_scale_gran gran, int compute_scale, void *workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return wa_kv_quant_fp8_fmt(x, xs, B, H, T_max, head_dim, lens, dst_start, cache, cs, cache_len,
                             scale, gran, WA_FP8_E4M3, compute_scale, workspace, workspace_bytes,
                             stream);
}

wa_status wa_kv_dequant_fp8(const uint8_t *cache, wa_strides cs, int cache_len,
                            const float *scale, wa_scale_gran gran, wa_fp8_format fmt,
                            const int32_t *lens, int B, int H, int T_max, int head_dim,
                            uint16_t *x, wa_strides xs, hipStream_t stream) {
  if (!cache || !scale || !x) return WA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || T_max <= 0 || cache_len <= 0) return WA_ERR_INVALID_ARGUMENT;
  if (gran != WA_SCALE_PER_TENSOR && gran != WA_SCALE_PER_HEAD) return WA_ERR_INVALID_ARGUMENT;
  if (fmt != WA_FP8_E4M3 && fmt != WA_FP8_E5M2) return WA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64) return WA_ERR_UNSUPPORTED;
  if (B > 65535 || H > 65535) return WA_ERR_UNSUPPORTED;
  if (!bf16_layout_ok(x, xs) || !u8_layout_ok(cache, cs)) return WA_ERR_UNSUPPORTED;
  wa_status st = check_device();
  if (st != WA_OK) return st;
  return from_hip(wa::launch_kv_dequant(cache, cs, cache_len, scale, gran == WA_SCALE_PER_HEAD,
                                        fmt == WA_FP8_E4M3 ? wa::Fp8::E4M3 : wa::Fp8::E5M2, lens,
                                        B, H, T_max, x, xs, stream));
}

wa_status wa_encoder_attn(const uint16_t *q, wa_strides qs, const uint16_t *k, wa_strides ks,
                          const uint16_t *v, wa_strides vs, uint16_t *o, wa_strides os, int B,
                          int H, int T_max, int head_dim, const int32_t *lens, int causal,
                          float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o) return WA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || T_max <= 0) return WA_ERR_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return WA_ERR_INVALID_ARGUMENT;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return WA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64) return WA_ERR_UNSUPPORTED;
  if (!bf16_layout_ok(q, qs) || !bf16_layout_ok(k, ks) || !bf16_layout_ok(v, vs) ||
      !bf16_layout_ok(o, os))
    return WA_ERR_UNSUPPORTED;
  if ((long)B * H * ((T_max + 127) / 128) > 0x7fffff00L) return WA_ERR_UNSUPPORTED;
  // the tile copies address a K or V row within a 64-row tile with a 32-bit
  // byte offset
  if (!tile_rows_fit(ks.t, 2) || !tile_rows_fit(vs.t, 2)) return WA_ERR_UNSUPPORTED;
  wa_status st = check_device();
  if (st != WA_OK) return st;
  return from_hip(wa::launch_encoder(q, qs, k, ks, v, vs, o, os, B, H, T_max, lens, T_max, lens,
                                     causal, softmax_scale, nullptr, nullptr, 0, stream));
}

wa_status wa_cross_attn(const uint16_t *q, wa_strides qs, const uint16_t *k, wa_strides ks,
                        const uint16_t *v, wa_strides vs, uint16_t *o, wa_strides os, int B, int H,
                        int T_q, int T_k, int head_dim, const int32_t *q_lens,
                        const int32_t *k_lens, float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o) return WA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || T_q <= 0 || T_k <= 0) return WA_ERR_INVALID_ARGUMENT;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return WA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64) return WA_ERR_UNSUPPORTED;
  if (!bf16_layout_ok(q, qs) || !bf16_layout_ok(k, ks) || !bf16_layout_ok(v, vs) ||
      !bf16_layout_ok(o, os))
    return WA_ERR_UNSUPPORTED;
  if ((long)B * H * ((T_q + 127) / 128) > 0x7fffff00L) return WA_ERR_UNSUPPORTED;
  if (!tile_rows_fit(ks.t, 2) || !tile_rows_fit(vs.t, 2)) return WA_ERR_UNSUPPORTED;
  wa_status st = check_device();
  if (st != WA_OK) return st;
  return from_hip(wa::launch_encoder(q, qs, k, ks, v, vs, o, os, B, H, T_q, q_lens, T_k, k_lens, 0,
                                     softmax_scale, nullptr, nullptr, 0, stream));
}

wa_status wa_encoder_attn_fp8qk(const uint8_t *q, wa_strides qs, const float *q_scale,
                                const uint8_t *k, wa_strides ks, const float *k_scale,
                                wa_scale_gran gran, const uint16_t *v, wa_strides vs, uint16_t *o,
                                wa_strides os, int B, int H, int T_max, int head_dim,
                                const int32_t *lens, int causal, float softmax_scale,
                                hipStream_t stream) {
  if (!q || !k || !v || !o || !q_scale || !k_scale) return WA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || T_max <= 0) return WA_ERR_INVALID_ARGUMENT;
  if (gran != WA_SCALE_PER_TENSOR && gran != WA_SCALE_PER_HEAD) return WA_ERR_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return WA_ERR_INVALID_ARGUMENT;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return WA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64) return WA_ERR_UNSUPPORTED;
  if (!u8_layout_ok(q, qs) || !u8_layout_ok(k, ks) || !bf16_layout_ok(v, vs) || !bf16_layout_ok(o, os))
    return WA_ERR_UNSUPPORTED;
  if ((long)B * H * ((T_max + 127) / 128) > 0x7fffff00L) return WA_ERR_UNSUPPORTED;
  if (!tile_rows_fit(ks.t, 1) || !tile_rows_fit(vs.t, 2)) return WA_ERR_UNSUPPORTED;
  wa_status st = check_device();
  if (st != WA_OK) return st;
  return from_hip(wa::launch_encoder(q, qs, k, ks, v, vs, o, os, B, H, T_max, lens, T_max, lens,
                                     causal, softmax_scale, q_scale, k_scale,
                                     gran == WA_SCALE_PER_HEAD, stream));
}

size_t wa_decode_attn_workspace_size(int B, int H, int cache_len) {
  if (B <= 0 || H <= 0 || cache_len <= 0) return 0;
  return wa::decode_workspace_bytes(B, H, wa::decode_plan(B, H, cache_len));
}

}  // extern "C"

namespace wa {

wa_status decode_args(const uint16_t *q, wa_strides qs, const uint8_t *k_cache,
                      const uint8_t *v_cache, wa_strides cs, int cache_len, const float *k_scale,
                      const float *v_scale, wa_scale_gran gran, const int32_t *lens, int B, int H,
                      int head_dim, float softmax_scale, const uint16_t *o, wa_strides os,
                      const uint16_t *k_new, const uint16_t *v_new, wa_strides ns, DecodeArgs *out) {
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !lens || !o)
    return WA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || cache_len <= 0) return WA_ERR_INVALID_ARGUMENT;
  if (gran != WA_SCALE_PER_TENSOR && gran != WA_SCALE_PER_HEAD) return WA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(softmax_scale)) return WA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64) return WA_ERR_UNSUPPORTED;
  const wa_strides qs2 = {qs.b, 0, qs.h}, os2 = {os.b, 0, os.h}, ns2 = {ns.b, 0, ns.h};
  if (!bf16_layout_ok(q, qs2) || !bf16_layout_ok(o, os2) || !u8_layout_ok(k_cache, cs) ||
      !u8_layout_ok(v_cache, cs))
    return WA_ERR_UNSUPPORTED;
  if (k_new && (!bf16_layout_ok(k_new, ns2) || !bf16_layout_ok(v_new, ns2))) return WA_ERR_UNSUPPORTED;
  if ((long)cache_len * cs.t > 0x7fffffffL) return WA_ERR_UNSUPPORTED;
  const DecodePlan plan = decode_plan(B, H, cache_len);
  if ((long)B * H * plan.n_split > 0x7fffff00L) return WA_ERR_UNSUPPORTED;
  out->plan = plan;
  out->qs = qs2;
  out->os = os2;
  out->ns = ns2;
  out->need = decode_workspace_bytes(B, H, plan);
  return WA_OK;
}

}  // namespace wa

namespace {

wa_status decode_common(const uint16_t *q, wa_strides qs, const uint8_t *k_cache,
                        const uint8_t *v_cache, wa_strides cs, int cache_len,
                        const float *k_scale, const float *v_scale, wa_scale_gran gran,
                        const int32_t *lens, int B, int H, int head_dim, float softmax_scale,
                        uint16_t *o, wa_strides os, void *workspace, size_t workspace_bytes,
                        hipStream_t stream, const uint16_t *k_new, const uint16_t *v_new,
                        wa_strides ns) {
  wa::DecodeArgs a;
  wa_status st = wa::decode_args(q, qs, k_cache, v_cache, cs, cache_len, k_scale, v_scale, gran, lens,
                                 B, H, head_dim, softmax_scale, o, os, k_new, v_new, ns, &a);
  if (st != WA_OK) return st;
  if (a.need > 0) {
    if (!workspace) return WA_ERR_INVALID_ARGUMENT;
    if (!aligned16(workspace)) return WA_ERR_UNSUPPORTED;
    if (workspace_bytes < a.need) return WA_ERR_WORKSPACE_TOO_SMALL;
  }
  st = wa::check_device();
  if (st != WA_OK) return st;
  return from_hip(wa::launch_decode(q, a.qs, k_cache, v_cache, cs, cache_len, k_scale, v_scale,
                                    gran == WA_SCALE_PER_HEAD, lens, B, H, softmax_scale, o, a.os,
                                    static_cast<float *>(workspace), a.plan, stream, k_new, v_new,
                                    a.ns));
}

}  // namespace

extern "C" {

wa_status wa_decode_attn(const uint16_t *q, wa_strides qs, const uint8_t *k_cache,
                         const uint8_t *v_cache, wa_strides cs, int cache_len,
                         const float *k_scale, const float *v_scale, wa_scale_gran gran,
                         const int32_t *lens, int B, int H, int head_dim, float softmax_scale,
                         uint16_t *o, wa_strides os, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  return decode_common(q, qs, k_cache, v_cache, cs, cache_len, k_scale, v_scale, gran, lens, B,
                       H, head_dim, softmax_scale, o, os, workspace, workspace_bytes, stream,
                       nullptr, nullptr, wa_strides{0, 0, 0});
}

wa_status wa_decode_attn_append(const uint16_t *q, wa_strides qs, const uint16_t *k_new,
                                const uint16_t *v_new, wa_strides ns, uint8_t *k_cache,
                                uint8_t *v_cache, wa_strides cs, int cache_len,
                                const float *k_scale, const float *v_scale, wa_scale_gran gran,
                                const int32_t *lens, int B, int H, int head_dim,
                                float softmax_scale, uint16_t *o, wa_strides os, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (!k_new || !v_new) return WA_ERR_INVALID_ARGUMENT;
  return decode_common(q, qs, k_cache, v_cache, cs, cache_len, k_scale, v_scale, gran, lens, B,
                       H, head_dim, softmax_scale, o, os, workspace, workspace_bytes, stream,
                       k_new, v_new, ns);
}

}  // extern "C"
