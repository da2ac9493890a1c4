// One-token decoder attention against an OCP E4M3 KV cache, for gfx950.
//
// The decoder self-attention (causal: the new token sees every cached slot)
// and cross-attention (no mask, 1500 encoder frames) of whisper-blaze 0.1.8
// ("Direct Kernel API"), reading the one-byte float8 cache that the HF blog
// "Blazingly fast whisper transcriptions with Inference Endpoints" (section
// "Inference Stack") describes, with fp32 arithmetic on dequantized values.
//
// HBM-bound design:
//   * grid = (b, h, key chunk); a block of 4 waves owns one chunk of one
//     (b, h); waves take 64-key blocks round robin.
//   * lane l of a wave reads 16 bytes (16 dims) of key row l/4 of each
//     16-key group: one dwordx4 load instruction moves 1 KB of contiguous
//     cache, and K and V of a 64-key block are 8 such loads per lane, all
//     issued before any use.
//   * dequantization is in registers (hardware fp8 -> fp32 pair converts);
//     the per-head key scale, the softmax scale and log2(e) are folded into
//     the query once, so a score is 16 FMAs plus a 4-lane DPP sum.
//   * online softmax per wave in the exp2 domain; the 4 waves merge in LDS;
//     chunks of one (b, h) merge in a second small kernel (skipped when a
//     (b, h) has one chunk).
#include <algorithm>
#include <cmath>

#include "wa_internal.h"

namespace wa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockKeys = 64;       // keys per wave iteration
constexpr int kPartialStride = 68;   // o[64], m, l, pad
constexpr float kLog2e = 1.4426950408889634f;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
// butterfly partners inside a quad: lane^1, lane^2
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  return v;
}
__device__ __forceinline__ float xor_shfl(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ void dequant16(const uint4 &c, float (&f)[16]) {
  uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    f[4 * i + 0] = lo[0];
    f[4 * i + 1] = lo[1];
    f[4 * i + 2] = hi[0];
    f[4 * i + 3] = hi[1];
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  // round to nearest even (inputs are finite)
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(kThreads) void decode_partial_kernel(
    const uint16_t *__restrict__ q, wa_strides qs, const uint8_t *__restrict__ kc,
    const uint8_t *__restrict__ vc, wa_strides cs, int cache_len, const float *__restrict__ ksc,
    const float *__restrict__ vsc, int per_head, const int32_t *__restrict__ lens, int H,
    float qmul, int chunk, int n_split, float *__restrict__ ws, uint16_t *__restrict__ o,
    wa_strides os) {
  __shared__ float s_o[kWaves][64];
  __shared__ float s_m[kWaves], s_l[kWaves];

  const int split = blockIdx.x % n_split;
  const int bh = blockIdx.x / n_split;
  const int b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane >> 2, qd = lane & 3;
  const int g = per_head ? h : 0;

  const int n = min(max(lens[b], 0), cache_len);
  const int j0 = split * chunk;
  const int j1 = min(j0 + chunk, n);

  // query slice (dims qd*16 .. qd*16+15), pre-multiplied by
  // softmax_scale * k_scale * log2(e) so scores come out in the exp2 domain
  float qf[16];
  {
    const float mul = qmul * ksc[g];
    const uint4 *qp = reinterpret_cast<const uint4 *>(q + (long)b * qs.b + (long)h * qs.h + qd * 16);
    uint4 a = qp[0], c = qp[1];
    uint32_t wq[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qf[2 * i] = __uint_as_float(wq[i] << 16) * mul;
      qf[2 * i + 1] = __uint_as_float(wq[i] & 0xffff0000u) * mul;
    }
  }

  const long base = (long)b * cs.b + (long)h * cs.h + qd * 16;
  const uint8_t *kb = kc + base;
  const uint8_t *vb = vc + base;

  float m = -INFINITY, l = 0.f;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  for (int blk = j0 + w * kBlockKeys; blk < j1; blk += kWaves * kBlockKeys) {
    uint4 kk[4], vv[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = blk + i * 16 + r;
      ok[i] = j < j1;
      if (ok[i]) {
        kk[i] = *reinterpret_cast<const uint4 *>(kb + (long)j * cs.t);
        vv[i] = *reinterpret_cast<const uint4 *>(vb + (long)j * cs.t);
      } else {
        kk[i] = make_uint4(0, 0, 0, 0);
        vv[i] = make_uint4(0, 0, 0, 0);
      }
    }
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float f[16];
      dequant16(kk[i], f);
      float acc_s = 0.f;
#pragma unroll
      for (int d = 0; d < 16; ++d) acc_s = fmaf(qf[d], f[d], acc_s);
      acc_s = quad_sum(acc_s);
      s[i] = ok[i] ? acc_s : -INFINITY;
    }
    float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    bm = fmaxf(bm, xor_shfl(bm, 4));
    bm = fmaxf(bm, xor_shfl(bm, 8));
    bm = fmaxf(bm, xor_shfl(bm, 16));
    bm = fmaxf(bm, xor_shfl(bm, 32));
    const float m_new = fmaxf(m, bm);          // finite: key blk is valid
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first block
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
    l = l * alpha + (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float f[16];
      dequant16(vv[i], f);
#pragma unroll
      for (int d = 0; d < 16; ++d) acc[d] = fmaf(p[i], f[d], acc[d]);
    }
    m = m_new;
  }

  // fold the 16 key rows of the wave (lanes with equal qd)
  l += xor_shfl(l, 4);
  l += xor_shfl(l, 8);
  l += xor_shfl(l, 16);
  l += xor_shfl(l, 32);
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    float v = acc[d];
    v += xor_shfl(v, 4);
    v += xor_shfl(v, 8);
    v += xor_shfl(v, 16);
    v += xor_shfl(v, 32);
    acc[d] = v;
  }
  if (r == 0) {
#pragma unroll
    for (int d = 0; d < 16; ++d) s_o[w][qd * 16 + d] = acc[d];
  }
  if (lane == 0) {
    s_m[w] = m;
    s_l[w] = l;
  }
  __syncthreads();
  if (w != 0) return;

  // merge the 4 waves: lane = output dim
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) M = fmaxf(M, s_m[i]);
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const float e = s_m[i] == -INFINITY ? 0.f : exp2f(s_m[i] - M);
      num = fmaf(e, s_o[i][lane], num);
      den = fmaf(e, s_l[i], den);
    }
  }
  if (n_split == 1) {
    const float out = den > 0.f ? num / den * vsc[g] : 0.f;
    o[(long)b * os.b + (long)h * os.h + lane] = f32_to_bf16(out);
  } else {
    float *pw = ws + ((long)split * (gridDim.x / n_split) + bh) * kPartialStride;
    pw[lane] = num;
    if (lane == 0) {
      pw[64] = M;
      pw[65] = den;
    }
  }
}

// Combine the chunk partials of one (b, h): with M the largest chunk max,
// o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i, times the value scale.
__global__ __launch_bounds__(64) void decode_merge_kernel(const float *__restrict__ ws, int BH,
                                                          int H, int n_split,
                                                          const float *__restrict__ vsc,
                                                          int per_head, uint16_t *__restrict__ o,
                                                          wa_strides os) {
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const int lane = threadIdx.x;
  float M = -INFINITY;
  for (int i = 0; i < n_split; ++i) M = fmaxf(M, ws[((long)i * BH + bh) * kPartialStride + 64]);
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int i = 0; i < n_split; ++i) {
      const float *pw = ws + ((long)i * BH + bh) * kPartialStride;
      const float mi = pw[64];
      const float e = mi == -INFINITY ? 0.f : exp2f(mi - M);
      num = fmaf(e, pw[lane], num);
      den = fmaf(e, pw[65], den);
    }
  }
  const float out = den > 0.f ? num / den * vsc[per_head ? h : 0] : 0.f;
  o[(long)b * os.b + (long)h * os.h + lane] = f32_to_bf16(out);
}

}  // namespace

DecodePlan decode_plan(int B, int H, int cache_len) {
  // Aim for about 2048 blocks (8 per CU) so every CU has loads in flight;
  // a chunk holds at least 256 keys (one 64-key block per wave).
  const long bh = (long)B * H;
  const int max_split = std::max(1, (cache_len + 255) / 256);
  int want = (int)std::min<long>(max_split, std::max<long>(1, (2048 + bh - 1) / bh));
  int chunk = (cache_len + want - 1) / want;
  chunk = ((chunk + kBlockKeys - 1) / kBlockKeys) * kBlockKeys;
  chunk = std::max(chunk, 256);
  DecodePlan p;
  p.chunk = chunk;
  p.n_split = std::max(1, (cache_len + chunk - 1) / chunk);
  return p;
}

size_t decode_workspace_bytes(int B, int H, const DecodePlan &p) {
  if (p.n_split <= 1) return 0;
  return (size_t)p.n_split * B * H * kPartialStride * sizeof(float);
}

hipError_t launch_decode(const uint16_t *q, wa_strides qs, const uint8_t *kc, const uint8_t *vc,
                         wa_strides cs, int cache_len, const float *k_scale,
                         const float *v_scale, int per_head, const int32_t *lens, int B, int H,
                         float softmax_scale, uint16_t *o, wa_strides os, float *ws,
                         const DecodePlan &plan, hipStream_t stream) {
  const int BH = B * H;
  hipLaunchKernelGGL(decode_partial_kernel, dim3(BH * plan.n_split), dim3(kThreads), 0, stream,
                     q, qs, kc, vc, cs, cache_len, k_scale, v_scale, per_head, lens, H,
                     softmax_scale * kLog2e, plan.chunk, plan.n_split, ws, o, os);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.n_split == 1) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(BH), dim3(64), 0, stream, ws, BH, H, plan.n_split,
                     v_scale, per_head, o, os);
  return hipGetLastError();
}

}  // namespace wa
