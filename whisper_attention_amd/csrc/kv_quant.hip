// bf16 -> OCP E4M3 KV-cache quantization for gfx950.
//
// The dynamic per-tensor / per-head scaling of whisper-blaze 0.1.8 (PyPI
// page, "Direct Kernel API": quantise_e4m3 returns codes and a scale) applied
// to the KV cache that the HF blog "Blazingly fast whisper transcriptions
// with Inference Endpoints" (section "Inference Stack") stores in one byte.
//
// Grid shape shared by the two streaming kernels: block (b, c) covers rows
// t in [c*kRows, (c+1)*kRows) of sequence b, clipped to lens[b] (one scalar
// load per block; blocks past the length exit at once).  A row is H*64 bf16,
// split into H*8 pieces of 16 bytes; thread p of a block owns piece p of
// every row it visits, so its head -- and its scale group -- never changes.
//
//   kv_amax_kernel      register max of |bits & 0x7fff| per thread (an exact,
//                       order-free integer max equal to the fp32 abs-max of
//                       the bf16 values), folded per group in LDS and stored
//                       as one partial per block and group.
//   kv_scale_kernel     one block folds the partials and writes
//                       scale[g] = amax_g / 448 (1 when amax_g is 0).
//   kv_encode_kernel    reads scale[g]; each thread divides its 8 values by
//                       it (IEEE fp32 division), clamps to +-448, converts with
//                       the hardware OCP fp8 conversion (round to nearest
//                       even) and writes 8 code bytes into the cache slot.
#include <algorithm>

#include "wa_internal.h"

namespace wa {
namespace {

constexpr int kRows = 32;       // rows of one sequence per block
constexpr int kUnroll = 8;      // loads in flight per thread

__device__ __forceinline__ uint32_t maxabs_bits8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, w[i] & 0x7fffu);
    m = max(m, (w[i] >> 16) & 0x7fffu);
  }
  return m;
}

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

__device__ __forceinline__ int seq_len(const int32_t *lens, int b, int T_max) {
  const int n = lens ? lens[b] : T_max;
  return min(max(n, 0), T_max);
}

__global__ __launch_bounds__(1024) void kv_amax_kernel(const uint16_t *__restrict__ x,
                                                       wa_strides xs, int T_max, int P,
                                                       const int32_t *__restrict__ lens,
                                                       int per_head, int groups,
                                                       uint32_t *__restrict__ partial) {
  extern __shared__ uint32_t smax[];  // [groups]
  const int b = blockIdx.x;
  const int t0 = blockIdx.y * kRows;
  const int t1 = min(t0 + kRows, seq_len(lens, b, T_max));
  const long blk = (long)blockIdx.y * gridDim.x + blockIdx.x;
  for (int g = threadIdx.x; g < groups; g += blockDim.x) smax[g] = 0;
  __syncthreads();
  if (t0 < t1) {
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
      const uint16_t *xp = x + (long)b * xs.b + (long)(p >> 3) * xs.h + (p & 7) * 8;
      uint32_t m = 0;
      for (int t = t0; t < t1; t += kUnroll) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          v[u] = t + u < t1 ? *reinterpret_cast<const uint4 *>(xp + (long)(t + u) * xs.t)
                            : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) m = max(m, maxabs_bits8(v[u]));
      }
      atomicMax(&smax[per_head ? (p >> 3) : 0], m);
    }
  }
  __syncthreads();
  for (int g = threadIdx.x; g < groups; g += blockDim.x) partial[blk * groups + g] = smax[g];
}

__global__ __launch_bounds__(1024) void kv_scale_kernel(const uint32_t *__restrict__ partial,
                                                        int n_blocks, int groups,
                                                        float *__restrict__ scale) {
  extern __shared__ uint32_t smax[];  // [groups]
  for (int g = threadIdx.x; g < groups; g += blockDim.x) smax[g] = 0;
  __syncthreads();
  if (groups <= (int)blockDim.x) {
    // thread -> one group and a strided subset of the blocks' partials
    const int per = blockDim.x / groups;
    if ((int)threadIdx.x < per * groups) {
      const int g = threadIdx.x % groups;
      uint32_t m = 0;
      for (long j = threadIdx.x / groups; j < n_blocks; j += per) m = max(m, partial[j * groups + g]);
      atomicMax(&smax[g], m);
    }
  } else {
    for (int g = threadIdx.x; g < groups; g += blockDim.x) {
      uint32_t m = 0;
      for (long j = 0; j < n_blocks; ++j) m = max(m, partial[j * groups + g]);
      smax[g] = m;
    }
  }
  __syncthreads();
  for (int g = threadIdx.x; g < groups; g += blockDim.x) {
    const float a = __uint_as_float(smax[g] << 16);  // bf16 bits -> fp32, exact
    scale[g] = a == 0.0f ? 1.0f : a / 448.0f;
  }
}

__global__ __launch_bounds__(1024) void kv_encode_kernel(
    const uint16_t *__restrict__ x, wa_strides xs, int T_max, int P,
    const int32_t *__restrict__ lens, const int32_t *__restrict__ dst_start,
    uint8_t *__restrict__ cache, wa_strides cs, int cache_len, const float *__restrict__ scale,
    int per_head) {
  const int b = blockIdx.x;
  const int t0 = blockIdx.y * kRows;
  const int t1 = min(t0 + kRows, seq_len(lens, b, T_max));
  if (t0 >= t1) return;
  const int d0 = dst_start ? dst_start[b] : 0;
  // slots outside [0, cache_len) are skipped
  const int ta = max(t0, -d0), tb = min(t1, cache_len - d0);
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int h = p >> 3;
    const float s = scale[per_head ? h : 0];
    const uint16_t *xp = x + (long)b * xs.b + (long)h * xs.h + (p & 7) * 8;
    uint8_t *cp = cache + (long)b * cs.b + (long)h * cs.h + (long)d0 * cs.t + (p & 7) * 8;
    for (int t = ta; t < tb; t += kUnroll) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (t + u < tb) v[u] = *reinterpret_cast<const uint4 *>(xp + (long)(t + u) * xs.t);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (t + u < tb) *reinterpret_cast<uint2 *>(cp + (long)(t + u) * cs.t) = encode8(v[u], s);
    }
  }
}

int block_threads(int P) { return std::min(1024, ((P + 63) / 64) * 64); }

}  // namespace

QuantPlan quant_plan(int B, int H, int T_max, wa_scale_gran gran) {
  QuantPlan p;
  p.pieces_per_row = H * 8;
  p.groups = gran == WA_SCALE_PER_HEAD ? H : 1;
  p.row_chunks = (T_max + kRows - 1) / kRows;
  p.blocks = (long)B * p.row_chunks;
  p.threads = block_threads(p.pieces_per_row);
  return p;
}

size_t quant_workspace_bytes(const QuantPlan &p) {
  const size_t n = (size_t)p.blocks * p.groups * sizeof(uint32_t);
  return (n + 255) & ~(size_t)255;
}

hipError_t launch_kv_quant(const uint16_t *x, wa_strides xs, int B, int H, int T_max,
                           const int32_t *lens, const int32_t *dst_start, uint8_t *cache,
                           wa_strides cs, int cache_len, float *scale, int per_head,
                           int compute_scale, uint32_t *ws, const QuantPlan &plan,
                           hipStream_t stream) {
  (void)H;
  const dim3 grid(B, plan.row_chunks);
  const size_t lds = (size_t)plan.groups * sizeof(uint32_t);
  if (compute_scale) {
    hipLaunchKernelGGL(kv_amax_kernel, grid, dim3(plan.threads), lds, stream, x, xs, T_max,
                       plan.pieces_per_row, lens, per_head, plan.groups, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kv_scale_kernel, dim3(1), dim3(1024), lds, stream, ws, (int)plan.blocks,
                       plan.groups, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kv_encode_kernel, grid, dim3(plan.threads), 0, stream, x, xs, T_max,
                     plan.pieces_per_row, lens, dst_start, cache, cs, cache_len, scale, per_head);
  return hipGetLastError();
}

}  // namespace wa
