// One-token decoder attention against an OCP E4M3 KV cache, for gfx950.
//
// The decoder self-attention (causal: the new token sees every cached slot)
// and cross-attention (no mask, 1500 encoder frames) of whisper-blaze 0.1.8
// ("Direct Kernel API"), reading the one-byte float8 cache that the HF blog
// "Blazingly fast whisper transcriptions with Inference Endpoints" (section
// "Inference Stack") describes, with fp32 arithmetic on dequantized values.
//
// HBM-bound design:
//   * one block per (b, h) and key chunk; its W waves (1 to 8, chosen so the
//     whole grid is resident at once, without a partly filled second round)
//     take 64-key blocks round robin.  A chunk is the whole cache unless
//     there are too few (b, h) pairs to fill the GPU.
//   * lane l of a wave reads 16 bytes (16 dims) of key row l/4 of each
//     16-key group: one dwordx4 load instruction moves 1 KB of contiguous
//     cache, and K and V of a 64-key block are 8 such loads per lane, all
//     issued before any use.  Rows past the length are never read (a lane
//     past the end re-reads the last valid row, whose weight it zeroes).
//   * dequantization is in registers (hardware fp8 -> fp32 pair converts);
//     the per-head key scale, the softmax scale and log2(e) are folded into
//     the query once, so a score is 16 FMAs plus a 4-lane DPP sum.
//   * online softmax per wave in the exp2 domain, with cross-lane maxima and
//     sums on DPP row rotations and the permlane16/32 swaps (no LDS round
//     trips); the W waves merge in LDS; the chunks of one (b, h), when there
//     are several, are merged by whichever chunk block finishes last (a
//     ticket on a per-(b, h) counter), in the same launch.
#include <algorithm>
#include <cmath>

#include "fp8_encode.h"
#include "wa_internal.h"

namespace wa {
namespace {

constexpr int kMaxWaves = 8;
constexpr int kBlockKeys = 64;       // keys per wave iteration
constexpr int kPartialStride = 68;   // o[64], m, l, pad
// Split-key workspace: a fixed block of uint32 counters, one per (b, h),
// then the partials.  The planner splits only below kSplitPairs (b, h)
// pairs, so the counters always fit and always sit at the same place: a
// workspace reused for calls of other shapes finds zeros there (every call
// leaves its counters zero), never the partials of an earlier call.
constexpr int kSplitPairs = 640;
constexpr long kCounterWords = kSplitPairs;   // 2560 bytes
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaveSlots = 5120;     // resident waves: 256 CUs x 4 SIMDs x 5

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
// Fold the 16 lanes that share lane & 3 (the key rows of one dim slice):
// rotations by 4 and 8 inside each row of 16 lanes, then the row swaps.
__device__ __forceinline__ float rows_sum(float v) {
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = __int_as_float(a[0]) + __int_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}
__device__ __forceinline__ float rows_max(float v) {
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x128>(v));
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}

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

// Partials of split-key calls are stored and read with agent-scope atomic
// operations: the blocks of one (b, h) run on different XCDs, whose L2
// caches are not coherent with each other.
__device__ __forceinline__ void store_partial(float *p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_partial(const float *p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t *>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}

// Called by the one wave of a block that stored the block's partial: once
// its stores are complete it draws a ticket from the (b, h)'s counter, and
// the wave that draws the last of the n_split tickets combines the partials
// (lane = output dim): with M the largest chunk max,
// o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i, times the value scale.
// It then sets the counter back to zero.  No block waits for another.
__device__ __forceinline__ void merge_if_last(uint32_t *cnt, const float *part, int BH, int bh,
                                              int n_split, int lane, float vs_g, uint16_t *orow) {
  __builtin_amdgcn_s_waitcnt(0);
  uint32_t t = 0;
  if (lane == 0) t = __hip_atomic_fetch_add(&cnt[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  t = (uint32_t)__shfl((int)t, 0, 64);
  if (t != (uint32_t)(n_split - 1)) return;
  // lane i (and i + 64, ...) reads chunk i's max: the loads go out together
  float M = -INFINITY;
  for (int i = lane; i < n_split; i += 64)
    M = fmaxf(M, load_partial(part + ((long)i * BH + bh) * kPartialStride + 64));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int i0 = 0; i0 < n_split; i0 += 64) {
      // chunk i0 + lane's weight and sum, then each chunk's O, dim = lane
      const int i = i0 + lane;
      float e = 0.f, li = 0.f;
      if (i < n_split) {
        const float *pw = part + ((long)i * BH + bh) * kPartialStride;
        const float mi = load_partial(pw + 64);
        li = load_partial(pw + 65);
        e = mi == -INFINITY ? 0.f : exp2f(mi - M);
      }
      den = fmaf(e, li, den);
      const int n = min(64, n_split - i0);
      for (int j0 = 0; j0 < n; j0 += 8) {
        float ov[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = min(j0 + u, n - 1);
          ov[u] = load_partial(part + ((long)(i0 + j) * BH + bh) * kPartialStride + lane);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float ej = __shfl(e, min(j0 + u, n - 1), 64);
          if (j0 + u < n) num = fmaf(ej, ov[u], num);
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
  }
  const float out = den > 0.f ? num / den * vs_g : 0.f;
  orow[lane] = f32_to_bf16(out);
  if (lane == 0) __hip_atomic_store(&cnt[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// kAppend: the new token's K and V (bf16 k_new, v_new [B][H][64]) are
// encoded with the stored scales into slot lens[b] - 1 of the caches and
// attended to from registers; every other wave and block reads only the
// slots before it, so nothing reads the slot while it is written.
template <bool kAppend>
__global__ __launch_bounds__(kMaxWaves * 64) __attribute__((amdgpu_waves_per_eu(5))) void decode_partial_kernel(
    const uint16_t *__restrict__ q, wa_strides qs, const uint8_t *__restrict__ kc,
    const uint8_t *__restrict__ vc, wa_strides cs, int cache_len, const float *__restrict__ ksc,
    const float *__restrict__ vsc, int per_head, const int32_t *__restrict__ lens, int H,
    float qmul, int chunk, int n_split, float *__restrict__ ws, uint16_t *__restrict__ o,
    wa_strides os, const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    wa_strides ns) {
  __shared__ float s_o[kMaxWaves][64];
  __shared__ float s_m[kMaxWaves], s_l[kMaxWaves];

  const int n_waves = blockDim.x >> 6;
  const int split = blockIdx.x % n_split;
  const int bh = blockIdx.x / n_split;
  const int BH = gridDim.x / n_split;
  // split-key calls: the workspace holds a counter per (b, h), then the partials
  uint32_t *cnt = reinterpret_cast<uint32_t *>(ws);
  float *part = ws + kCounterWords;
  const int b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane >> 2, qd = lane & 3;
  const int g = per_head ? h : 0;

  const int n = min(max(lens[b], 0), cache_len);
  const int j0 = split * chunk;
  // with kAppend the last slot, n - 1, is the new token's, handled apart
  const int j1 = min(j0 + chunk, kAppend ? n - 1 : n);

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

  // wave-uniform bases, 32-bit per-lane offsets (the host checks that one
  // (b, h) slab spans less than 2^31 bytes)
  const long base = (long)b * cs.b + (long)h * cs.h;
  const uint8_t *kb = kc + base;
  const uint8_t *vb = vc + base;
  const uint32_t ts = (uint32_t)cs.t;

  float m = -INFINITY, l = 0.f;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  for (int blk = j0 + w * kBlockKeys; blk < j1; blk += n_waves * kBlockKeys) {
    uint4 kk[4], vv[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = blk + i * 16 + r;
      ok[i] = j < j1;
      const uint32_t off = (uint32_t)min(j, j1 - 1) * ts + qd * 16;  // past the end: last valid row
      kk[i] = load_stream(kb + off);
      vv[i] = load_stream(vb + off);
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
    const float bm = rows_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
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

  if (kAppend && w == 0 && n > 0 && (n - 1) / chunk == split) {
    // encode the new token's K and V rows into slot n - 1 (lanes 0..3 each
    // hold 16 dims), then one more online-softmax step with that row alone
    const int slot = n - 1;
    const float sk = ksc[g], sv = vsc[g];
    uint4 kn = make_uint4(0, 0, 0, 0), vn = make_uint4(0, 0, 0, 0);
    if (r == 0) {
      const long src = (long)b * ns.b + (long)h * ns.h + qd * 16;
      const uint4 *kp = reinterpret_cast<const uint4 *>(k_new + src);
      const uint4 *vp = reinterpret_cast<const uint4 *>(v_new + src);
      const uint2 k0 = encode8_scaled(kp[0], sk, 1.0f / sk, fast_scale(sk));
      const uint2 k1 = encode8_scaled(kp[1], sk, 1.0f / sk, fast_scale(sk));
      const uint2 v0 = encode8_scaled(vp[0], sv, 1.0f / sv, fast_scale(sv));
      const uint2 v1 = encode8_scaled(vp[1], sv, 1.0f / sv, fast_scale(sv));
      kn = make_uint4(k0.x, k0.y, k1.x, k1.y);
      vn = make_uint4(v0.x, v0.y, v1.x, v1.y);
      const long dst = (long)b * cs.b + (long)h * cs.h + (long)slot * cs.t + qd * 16;
      *reinterpret_cast<uint4 *>(const_cast<uint8_t *>(kc) + dst) = kn;
      *reinterpret_cast<uint4 *>(const_cast<uint8_t *>(vc) + dst) = vn;
    }
    float f[16];
    dequant16(kn, f);
    float sn = 0.f;
#pragma unroll
    for (int d = 0; d < 16; ++d) sn = fmaf(qf[d], f[d], sn);
    sn = quad_sum(sn);
    if (r != 0) sn = -INFINITY;
    const float m_new = fmaxf(m, rows_max(sn));
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    const float p = __builtin_amdgcn_exp2f(sn - m_new);   // 0 outside lanes 0..3
    l = l * alpha + p;
    dequant16(vn, f);
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] = fmaf(p, f[d], acc[d] * alpha);
    m = m_new;
  }

  // fold the 16 key rows of the wave (lanes with equal qd)
  l = rows_sum(l);
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] = rows_sum(acc[d]);
  const float vs_g = vsc[g];
  if (n_waves == 1) {
    // lanes 0..3 hold the whole result: dims qd*16 .. +16
    if (r == 0) {
      if (n_split == 1) {
        uint16_t *op = o + (long)b * os.b + (long)h * os.h + qd * 16;
        const float inv = l > 0.f ? vs_g / l : 0.f;
        uint32_t wd[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          wd[i] = (uint32_t)f32_to_bf16(acc[2 * i] * inv) | ((uint32_t)f32_to_bf16(acc[2 * i + 1] * inv) << 16);
        reinterpret_cast<uint4 *>(op)[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        reinterpret_cast<uint4 *>(op)[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
      } else {
        float *pw = part + ((long)split * BH + bh) * kPartialStride;
#pragma unroll
        for (int d = 0; d < 16; ++d) store_partial(pw + qd * 16 + d, acc[d]);
        if (qd == 0) {
          store_partial(pw + 64, m);
          store_partial(pw + 65, l);
        }
      }
    }
    if (n_split > 1) merge_if_last(cnt, part, BH, bh, n_split, lane, vs_g, o + (long)b * os.b + (long)h * os.h);
    return;
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

  // merge the waves: lane = output dim
  float M = -INFINITY;
  for (int i = 0; i < n_waves; ++i) M = fmaxf(M, s_m[i]);
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int i = 0; i < n_waves; ++i) {
      const float e = s_m[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[i] - M);
      num = fmaf(e, s_o[i][lane], num);
      den = fmaf(e, s_l[i], den);
    }
  }
  if (n_split == 1) {
    const float out = den > 0.f ? num / den * vs_g : 0.f;
    o[(long)b * os.b + (long)h * os.h + lane] = f32_to_bf16(out);
  } else {
    float *pw = part + ((long)split * BH + bh) * kPartialStride;
    store_partial(pw + lane, num);
    if (lane == 0) {
      store_partial(pw + 64, M);
      store_partial(pw + 65, den);
    }
    merge_if_last(cnt, part, BH, bh, n_split, lane, vs_g, o + (long)b * os.b + (long)h * os.h);
  }
}

}  // namespace

DecodePlan decode_plan(int B, int H, int cache_len) {
  // One wave per 64-key block at most, and a grid that fits in the resident
  // wave slots at once.  Enough (b, h) pairs: one chunk each, as many waves
  // per block as fit (up to 8).  Few pairs: split the keys into chunks of at
  // least 256 so the GPU still has about 1024 blocks of 4 waves.
  const long bh = (long)B * H;
  const int key_blocks = (cache_len + kBlockKeys - 1) / kBlockKeys;
  DecodePlan p;
  static_assert(kSplitPairs * 4 == kWaveSlots / 2, "the split threshold is the counters' count");
  if (bh >= kSplitPairs) {
    p.n_split = 1;
    p.chunk = key_blocks * kBlockKeys;
    p.waves = (int)std::max<long>(1, std::min<long>(std::min(kMaxWaves, key_blocks), kWaveSlots / bh));
    // a short cache (a decoder self-attention cache holds at most 448
    // tokens): one 64-key block per wave, so no wave waits for two loads in
    // a row; waves past a sequence's length exit at once
    return p;
  }
  const int max_split = std::max(1, (cache_len + 255) / 256);
  const int want = (int)std::min<long>(max_split, std::max<long>(1, (1024 + bh - 1) / bh));
  int chunk = (cache_len + want - 1) / want;
  chunk = ((chunk + kBlockKeys - 1) / kBlockKeys) * kBlockKeys;
  chunk = std::max(chunk, 256);
  p.chunk = chunk;
  p.n_split = std::max(1, (cache_len + chunk - 1) / chunk);
  p.waves = std::min(4, (chunk + kBlockKeys - 1) / kBlockKeys);
  return p;
}

size_t decode_workspace_bytes(int B, int H, const DecodePlan &p) {
  if (p.n_split <= 1) return 0;
  return (size_t)kCounterWords * 4 + (size_t)p.n_split * B * H * kPartialStride * sizeof(float);
}

hipError_t launch_decode(const uint16_t *q, wa_strides qs, const uint8_t *kc, const uint8_t *vc,
                         wa_strides cs, int cache_len, const float *k_scale,
                         const float *v_scale, int per_head, const int32_t *lens, int B, int H,
                         float softmax_scale, uint16_t *o, wa_strides os, float *ws,
                         const DecodePlan &plan, hipStream_t stream, const uint16_t *k_new,
                         const uint16_t *v_new, wa_strides ns) {
  const int BH = B * H;
  if (k_new)
    hipLaunchKernelGGL(decode_partial_kernel<true>, dim3(BH * plan.n_split), dim3(plan.waves * 64), 0,
                       stream, q, qs, kc, vc, cs, cache_len, k_scale, v_scale, per_head, lens, H,
                       softmax_scale * kLog2e, plan.chunk, plan.n_split, ws, o, os, k_new, v_new, ns);
  else
    hipLaunchKernelGGL(decode_partial_kernel<false>, dim3(BH * plan.n_split), dim3(plan.waves * 64), 0,
                       stream, q, qs, kc, vc, cs, cache_len, k_scale, v_scale, per_head, lens, H,
                       softmax_scale * kLog2e, plan.chunk, plan.n_split, ws, o, os, k_new, v_new, ns);
  return hipGetLastError();
}

}  // namespace wa
