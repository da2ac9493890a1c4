// bf16 -> OCP float8 encoding of 8 values (one 16-byte piece), E4M3 or E5M2,
// shared by the cache-fill kernels and the decode kernel that appends a
// token.  gfx950 device code; the library is built without fast-math and
// with correctly rounded fp32 division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wa {

enum class Fp8 : int { E4M3 = 0, E5M2 = 1 };

// Largest finite magnitude of each format: E4M3 1.75 * 2^8, E5M2 1.75 * 2^15.
template <Fp8 F> constexpr float fp8_max() { return F == Fp8::E4M3 ? 448.0f : 57344.0f; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <Fp8 F> __device__ __forceinline__ float clamp_max(float y) {
  return fminf(fmaxf(y, -fp8_max<F>()), fp8_max<F>());
}

// Two in-range fp32 values -> two codes in byte pair `hi` of `old`, with the
// hardware OCP conversion (round to nearest even).
template <Fp8 F, bool kHi> __device__ __forceinline__ int cvt_pk(float a, float b, int old) {
  if constexpr (F == Fp8::E4M3) return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, kHi);
  else return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, kHi);
}

template <Fp8 F> __device__ __forceinline__ uint2 pack8(const float (&y)[8]) {
  int lo = cvt_pk<F, false>(y[0], y[1], 0);
  lo = cvt_pk<F, true>(y[2], y[3], lo);
  int hi = cvt_pk<F, false>(y[4], y[5], 0);
  hi = cvt_pk<F, true>(y[6], y[7], hi);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// 8 bf16 -> 8 codes.  The quotient is the IEEE correctly rounded fp32
// division; the clamp makes the conversion saturate.
template <Fp8 F = Fp8::E4M3> __device__ __forceinline__ uint2 encode8(uint4 v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = clamp_max<F>(bf16_lo(w[i]) / s);
    y[2 * i + 1] = clamp_max<F>(bf16_hi(w[i]) / s);
  }
  return pack8<F>(y);
}

// The same 8 codes with the quotient from the reciprocal r = 1/s (IEEE) and
// one FMA correction (Markstein): q0 = |x|*r, e = |x| - q0*s (exact in one
// FMA), q = q0 + e*r rounded once.  For 2^-80 <= s <= 2^80 this gives the
// correctly rounded |x|/s wherever a code can be non-zero, and below that
// both quotients round to a zero code (checked for every finite bf16 x and
// every dynamic scale amax/FMAX in that range, for both formats); the sign
// is restored from x, so -0 stays -0.  q0 is clamped first so that no step
// overflows.
template <Fp8 F> __device__ __forceinline__ float quot_fast(float x, float s, float r) {
  const float a = fabsf(x);
  const float q0 = fminf(a * r, fp8_max<F>() + 1.0f);
  const float e = __builtin_fmaf(-q0, s, a);
  const float q = fminf(__builtin_fmaf(e, r, q0), fp8_max<F>());
  return __builtin_copysignf(q, x);
}

template <Fp8 F = Fp8::E4M3> __device__ __forceinline__ uint2 encode8_fast(uint4 v, float s, float r) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = quot_fast<F>(bf16_lo(w[i]), s, r);
    y[2 * i + 1] = quot_fast<F>(bf16_hi(w[i]), s, r);
  }
  return pack8<F>(y);
}

// The quotient of quot_fast without its clamps, for a dynamic scale: every
// value encoded with s = fp32(amax / FMAX) has |x| <= amax, so |x| * r and
// the corrected quotient stay within FMAX (1 + 2^-22) -- no step can
// overflow, and a quotient a rounding above FMAX still converts to the
// largest code, as the clamped one does.
template <Fp8 F> __device__ __forceinline__ float quot_dyn(float x, float s, float r) {
  const float a = fabsf(x);
  const float q0 = a * r;
  const float e = __builtin_fmaf(-q0, s, a);
  return __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
}

template <Fp8 F = Fp8::E4M3> __device__ __forceinline__ uint2 encode8_dyn(uint4 v, float s, float r) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = quot_dyn<F>(bf16_lo(w[i]), s, r);
    y[2 * i + 1] = quot_dyn<F>(bf16_hi(w[i]), s, r);
  }
  return pack8<F>(y);
}

__device__ __forceinline__ bool fast_scale(float s) { return s >= 0x1p-80f && s <= 0x1p80f; }

// x / s encoded, by whichever quotient path the scale allows (the two give
// the same codes; see quot_fast).
template <Fp8 F = Fp8::E4M3>
__device__ __forceinline__ uint2 encode8_scaled(uint4 v, float s, float rcp, bool fast) {
  return fast ? encode8_fast<F>(v, s, rcp) : encode8<F>(v, s);
}

}  // namespace wa
