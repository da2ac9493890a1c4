// bf16 -> OCP E4M3 encoding of 8 values (one 16-byte piece), shared by the
// cache-fill kernels and the decode kernel that appends a token.  gfx950
// device code; the library is built without fast-math and with correctly
// rounded fp32 division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wa {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float clamp448(float y) { return fminf(fmaxf(y, -448.0f), 448.0f); }

// 8 bf16 -> 8 E4M3 codes.  The quotient is the IEEE correctly rounded fp32
// division (the library is built without fast-math and with correctly
// rounded fp32 division); the clamp makes the conversion saturate.
__device__ __forceinline__ uint2 encode8(uint4 v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = clamp448(bf16_lo(w[i]) / s);
    y[2 * i + 1] = clamp448(bf16_hi(w[i]) / s);
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// The same 8 codes with the quotient from the reciprocal r = 1/s (IEEE) and
// one FMA correction (Markstein): q0 = |x|*r, e = |x| - q0*s (exact in one
// FMA), q = q0 + e*r rounded once.  For 2^-80 <= s <= 2^80 this gives the
// correctly rounded |x|/s wherever the quotient is at least 2^-12 -- every
// quotient that can encode to a non-zero code -- and below that both round
// to a zero code; the sign is restored from x, so -0 stays -0.  q0 is
// clamped first so that no step overflows.  Checked against IEEE division
// for every finite bf16 x and every dynamic scale amax/448 in that range.
__device__ __forceinline__ float quot_fast(float x, float s, float r) {
  const float a = fabsf(x);
  const float q0 = fminf(a * r, 449.0f);
  const float e = __builtin_fmaf(-q0, s, a);
  const float q = fminf(__builtin_fmaf(e, r, q0), 448.0f);
  return __builtin_copysignf(q, x);
}

__device__ __forceinline__ uint2 encode8_fast(uint4 v, float s, float r) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = quot_fast(bf16_lo(w[i]), s, r);
    y[2 * i + 1] = quot_fast(bf16_hi(w[i]), s, r);
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

__device__ __forceinline__ bool fast_scale(float s) { return s >= 0x1p-80f && s <= 0x1p80f; }

// x / s encoded, by whichever quotient path the scale allows (the two give
// the same codes; see quot_fast).
__device__ __forceinline__ uint2 encode8_scaled(uint4 v, float s, float rcp, bool fast) {
  return fast ? encode8_fast(v, s, rcp) : encode8(v, s);
}

}  // namespace wa
