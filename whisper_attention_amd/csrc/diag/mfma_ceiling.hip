// Matrix-core ceiling probe: waves that issue nothing but independent dense
// MFMA products, and read the shader clock and the constant clock around
// the loop, so that the attention kernels' rates can be set against what
// the GPU sustains under a matrix-core load at that moment.

#include <hip/hip_runtime.h>

#include "wa_diag.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 4;

template <bool kFp8>
__global__ __launch_bounds__(256) void mfma_ceiling_kernel(int iters, uint64_t *ticks) {
  const int lane = threadIdx.x & 63;
  // operands from the lane index, so nothing folds; small magnitudes keep
  // the sums finite over any number of iterations allowed
  bf16x8 a16, b16;
  i32x8 a8, b8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a16[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b16[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
    // E4M3 bytes 0x08..0x0F are subnormals below 2^-6
    a8[e] = 0x08090A0B + (lane & 3);
    b8[e] = 0x0C0D0E0F - (lane & 3);
  }
  f32x16 c[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) c[j] = f32x16{};
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t t0 = clock64(), r0 = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
      if (kFp8)
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c[j], 0, 0, 0, 0, 0, 0);
      else
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a16, b16, c[j], 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t t1 = clock64(), r1 = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc += c[j][e];
  if (threadIdx.x == 0) {
    // the comparison keeps the products live; it is false for these finite sums
    ticks[2 * blockIdx.x] = acc != acc ? 0 : t1 - t0;
    ticks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// One wave per block reads the shader clock (s_memtime) and the constant
// clock (s_memrealtime) over a spin of `spin` constant-clock ticks; the loop
// also ends after max_iters reads, so it ends even if the constant clock
// stood still.
__global__ __launch_bounds__(64) void sclk_probe_kernel(int spin, int max_iters, uint64_t *ticks) {
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t t0 = clock64(), r0 = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);
  uint64_t r1 = r0;
  for (int i = 0; i < max_iters && r1 - r0 < (uint64_t)spin; ++i) r1 = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t t1 = clock64();
  if (threadIdx.x == 0) {
    ticks[2 * blockIdx.x] = t1 - t0;
    ticks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

wa_status wa_diag_sclk_probe(int n_blocks, int spin, uint64_t *ticks, hipStream_t stream) {
  if (!ticks || n_blocks < 1 || n_blocks > (1 << 16) || spin < 1 || spin > 100000)
    return WA_ERR_INVALID_ARGUMENT;
  // one constant-clock read per iteration: 64 reads per tick leave the spin
  // the deciding condition at any clock rate this probe is for
  hipLaunchKernelGGL(sclk_probe_kernel, dim3(n_blocks), dim3(64), 0, stream, spin, spin * 64, ticks);
  return hipGetLastError() == hipSuccess ? WA_OK : WA_ERR_HIP;
}

wa_status wa_diag_mfma_ceiling(wa_diag_dtype dtype, int n_blocks, int iters, uint64_t *ticks,
                               hipStream_t stream) {
  if (!ticks || n_blocks < 1 || n_blocks > (1 << 20) || iters < 1 || iters > (1 << 20))
    return WA_ERR_INVALID_ARGUMENT;
  if (dtype != WA_DIAG_BF16 && dtype != WA_DIAG_FP8) return WA_ERR_INVALID_ARGUMENT;
  auto kernel = dtype == WA_DIAG_FP8 ? mfma_ceiling_kernel<true> : mfma_ceiling_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3(n_blocks), dim3(256), 0, stream, iters, ticks);
  return hipGetLastError() == hipSuccess ? WA_OK : WA_ERR_HIP;
}

wa_status wa_diag_wall_clock_khz(int *khz) {
  if (!khz) return WA_ERR_INVALID_ARGUMENT;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return WA_ERR_HIP;
  if (hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return WA_ERR_HIP;
  return WA_OK;
}

}  // extern "C"
