// Internal declarations shared by the wa_* host entry points and the kernel
// launchers.  gfx950 (CDNA4) only: wave64, MFMA 32x32x16 bf16, OCP fp8
// conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8_encode.h"
#include "wa.h"

namespace wa {

// A 16-byte load that is not kept in the last-level cache, for data read once
// (the cache codes that decode attention and the dequantise read): the
// last-level cache then keeps what the kernels before wrote instead of
// evicting -- and writing back -- it during these reads.  (The quantize's
// second read of its input stays cached: the prefill attention that follows
// reads the same K and V.)
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void *p) {
  const u32x4_nt v = __builtin_nontemporal_load(static_cast<const u32x4_nt *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---- kv quantize --------------------------------------------------------
struct QuantPlan {
  int pieces_per_row;   // H * 8: one piece = 8 bf16 = 16 bytes
  int groups;           // 1 (per tensor) or H (per head)
  int threads;          // threads per block
  int rows_per_pass;    // whole rows a block covers at once (0: threads loop over pieces)
  int amax_chunks;      // amax blocks per sequence (at most 32; they stride over longer sequences)
  int enc_chunks;       // encode blocks per sequence
  long blocks;          // amax blocks in all (B * amax_chunks): partials per group
};
QuantPlan quant_plan(int B, int H, int T_max, wa_scale_gran gran);
// per tensor: the counter and B * 32 partials per scale group, whatever T_max
size_t quant_workspace_bytes(int B, int groups);

// One or two tensors (K and V) that share shape, lengths, slots and the cache
// layout; each has its own input, cache and scales.
struct QuantTensors {
  const uint16_t *x[2];
  wa_strides xs[2];
  uint8_t *cache[2];
  float *scale[2];
};
// The workspace holds n_tensors * quant_workspace_bytes(B, plan.groups) bytes.
hipError_t launch_kv_quant(const QuantTensors &qt, int n_tensors, int B, int H, int T_max,
                           const int32_t *lens, const int32_t *dst_start, wa_strides cs,
                           int cache_len, int per_head, int compute_scale, Fp8 fmt, uint32_t *ws,
                           const QuantPlan &plan, hipStream_t stream);

// ---- dequantize -----------------------------------------------------------
hipError_t launch_kv_dequant(const uint8_t *cache, wa_strides cs, int cache_len, const float *scale,
                             int per_head, Fp8 fmt, const int32_t *lens, int B, int H, int T_max,
                             uint16_t *x, wa_strides xs, hipStream_t stream);

// ---- decode attention ---------------------------------------------------
struct DecodePlan {
  int n_split;          // key chunks per (b, h)
  int chunk;            // keys per chunk (multiple of 64)
  int waves;            // waves per block (1..8)
};
DecodePlan decode_plan(int B, int H, int cache_len);
size_t decode_workspace_bytes(int B, int H, const DecodePlan &p);

// Host-side checks of a decode call (wa_api.hip), shared by every decode
// entry point; nothing here touches the device.  On WA_OK, `out` holds the
// plan, the token strides with t zeroed, and the partials' byte count.
struct DecodeArgs {
  DecodePlan plan;
  wa_strides qs, os, ns;
  size_t need;
};
wa_status decode_args(const uint16_t *q, wa_strides qs, const uint8_t *k_cache,
                      const uint8_t *v_cache, wa_strides cs, int cache_len, const float *k_scale,
                      const float *v_scale, wa_scale_gran gran, const int32_t *lens, int B, int H,
                      int head_dim, float softmax_scale, const uint16_t *o, wa_strides os,
                      const uint16_t *k_new, const uint16_t *v_new, wa_strides ns, DecodeArgs *out);

// The first call on each device checks that it is a gfx950.
wa_status check_device();

hipError_t launch_decode(const uint16_t *q, wa_strides qs, const uint8_t *kc, const uint8_t *vc,
                         wa_strides cs, int cache_len, const float *k_scale,
                         const float *v_scale, int per_head, const int32_t *lens, int B, int H,
                         float softmax_scale, uint16_t *o, wa_strides os, float *ws,
                         const DecodePlan &plan, hipStream_t stream,
                         const uint16_t *k_new = nullptr, const uint16_t *v_new = nullptr,
                         wa_strides ns = wa_strides{0, 0, 0});

// ---- encoder / prefill attention ----------------------------------------
// q_scale == nullptr: bf16 Q and K.  Otherwise Q and K are E4M3 codes with
// those dequantization scales ([1], or [H] when per_head).  Queries
// i < q_lens[b] of Tq_max attend keys j < k_lens[b] of Tk_max (a null
// length array means the full size); causal needs the same sequence for both.
hipError_t launch_encoder(const void *q, wa_strides qs, const void *k, wa_strides ks,
                          const uint16_t *v, wa_strides vs, uint16_t *o, wa_strides os, int B,
                          int H, int Tq_max, const int32_t *q_lens, int Tk_max,
                          const int32_t *k_lens, int causal, float softmax_scale,
                          const float *q_scale, const float *k_scale, int per_head,
                          hipStream_t stream);

}  // namespace wa
