// bf16 -> OCP E4M3 KV-cache quantization for gfx950.
//
// The dynamic per-tensor / per-head scaling of whisper-blaze 0.1.8 (PyPI
// page, "Direct Kernel API": quantise_e4m3 returns codes and a scale) applied
// to the KV cache that the HF blog "Blazingly fast whisper transcriptions
// with Inference Endpoints" (section "Inference Stack") stores in one byte.
//
// Two HBM-bound passes:
//   1. kv_amax_kernel: every thread owns one fixed 16-byte piece position of
//      a row (so one fixed head) and keeps a register max of |bits & 0x7fff|
//      over the rows it visits -- an exact, order-free integer max that
//      equals the fp32 abs-max of the bf16 values.  Each block folds its
//      threads into per-group maxima in LDS and writes them to the workspace.
//   2. kv_encode_kernel: each block first folds the per-block maxima into
//      the group scales (block 0 also stores them), then every thread
//      divides its 8 values by the scale (IEEE fp32 division), clamps to
//      +-448 and converts with the hardware OCP fp8 conversion
//      (round-to-nearest-even), writing 8 code bytes to the cache slot.
//
// The total thread count of both grids is a multiple of the number of
// pieces per row, so the piece (and head) of a thread never changes while it
// strides over rows.
#include <algorithm>

#include "wa_internal.h"

namespace wa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsUnroll = 4;

__device__ __forceinline__ uint32_t maxabs_bits8(uint4 v) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
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

__device__ __forceinline__ float clamp448(float y) {
  return fminf(fmaxf(y, -448.0f), 448.0f);
}

// 8 bf16 -> 8 E4M3 codes (RNE, saturated by the clamp).  The division is
// the IEEE correctly rounded fp32 quotient (the library is built without
// fast-math and with correctly rounded fp32 division).
__device__ __forceinline__ uint2 encode8(uint4 v, float s) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
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
  int n = lens ? lens[b] : T_max;
  return min(max(n, 0), T_max);
}

__global__ __launch_bounds__(kThreads) void kv_amax_kernel(
    const uint16_t *__restrict__ x, wa_strides xs, int B, int T_max, int P,
    const int32_t *__restrict__ lens, int per_head, int groups, uint32_t *__restrict__ partial) {
  extern __shared__ uint32_t smax[];  // [groups]
  for (int g = threadIdx.x; g < groups; g += kThreads) smax[g] = 0;
  __syncthreads();

  const long gtid = (long)blockIdx.x * kThreads + threadIdx.x;
  const long TT = (long)gridDim.x * kThreads;
  const int p = (int)(gtid % P);
  const int h = p >> 3;
  const int d0 = (p & 7) * 8;
  const long rstride = TT / P;  // exact: TT is a multiple of P
  const long nrows = (long)B * T_max;
  const uint16_t *xh = x + (long)h * xs.h + d0;

  uint32_t m = 0;
  for (long row = gtid / P; row < nrows; row += kRowsUnroll * rstride) {
    uint4 v[kRowsUnroll];
    bool ok[kRowsUnroll];
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) {
      long r = row + u * rstride;
      int b = (int)(r / T_max);
      int t = (int)(r - (long)b * T_max);
      ok[u] = r < nrows && t < seq_len(lens, b, T_max);
      if (ok[u]) v[u] = *reinterpret_cast<const uint4 *>(xh + (long)b * xs.b + (long)t * xs.t);
    }
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u)
      if (ok[u]) m = max(m, maxabs_bits8(v[u]));
  }
  atomicMax(&smax[per_head ? h : 0], m);
  __syncthreads();
  for (int g = threadIdx.x; g < groups; g += kThreads)
    partial[(long)blockIdx.x * groups + g] = smax[g];
}

__global__ __launch_bounds__(kThreads) void kv_encode_kernel(
    const uint16_t *__restrict__ x, wa_strides xs, int B, int T_max, int P,
    const int32_t *__restrict__ lens, const int32_t *__restrict__ dst_start,
    uint8_t *__restrict__ cache, wa_strides cs, int cache_len, float *__restrict__ scale,
    int per_head, int groups, int compute_scale, const uint32_t *__restrict__ partial,
    int amax_blocks) {
  extern __shared__ uint32_t smax[];  // [groups]
  const long gtid = (long)blockIdx.x * kThreads + threadIdx.x;
  const long TT = (long)gridDim.x * kThreads;
  const int p = (int)(gtid % P);
  const int h = p >> 3;
  const int d0 = (p & 7) * 8;
  const int g = per_head ? h : 0;

  float s;
  if (compute_scale) {
    for (int i = threadIdx.x; i < groups; i += kThreads) smax[i] = 0;
    __syncthreads();
    const long n = (long)amax_blocks * groups;
    for (long i = threadIdx.x; i < n; i += kThreads) atomicMax(&smax[i % groups], partial[i]);
    __syncthreads();
    // amax as fp32 (bf16 bits shifted into place), scale = amax / 448
    const float amax = __uint_as_float(smax[g] << 16);
    s = amax == 0.0f ? 1.0f : amax / 448.0f;
    if (blockIdx.x == 0) {
      for (int i = threadIdx.x; i < groups; i += kThreads) {
        const float a = __uint_as_float(smax[i] << 16);
        scale[i] = a == 0.0f ? 1.0f : a / 448.0f;
      }
    }
  } else {
    s = scale[g];
  }

  const long rstride = TT / P;
  const long nrows = (long)B * T_max;
  const uint16_t *xh = x + (long)h * xs.h + d0;
  uint8_t *ch = cache + (long)h * cs.h + d0;
  for (long row = gtid / P; row < nrows; row += kRowsUnroll * rstride) {
    uint4 v[kRowsUnroll];
    long dst[kRowsUnroll];
    bool ok[kRowsUnroll];
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) {
      long r = row + u * rstride;
      int b = (int)(r / T_max);
      int t = (int)(r - (long)b * T_max);
      ok[u] = false;
      if (r < nrows && t < seq_len(lens, b, T_max)) {
        int slot = (dst_start ? dst_start[b] : 0) + t;
        if (slot >= 0 && slot < cache_len) {
          ok[u] = true;
          dst[u] = (long)b * cs.b + (long)slot * cs.t;
          v[u] = *reinterpret_cast<const uint4 *>(xh + (long)b * xs.b + (long)t * xs.t);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u)
      if (ok[u]) *reinterpret_cast<uint2 *>(ch + dst[u]) = encode8(v[u], s);
  }
}

int round_to_unit(int want, int unit) { return std::max(unit, (want / unit) * unit); }

}  // namespace

QuantPlan quant_plan(int B, int H, int T_max, wa_scale_gran gran) {
  QuantPlan p;
  p.pieces_per_row = H * 8;
  p.groups = gran == WA_SCALE_PER_HEAD ? H : 1;
  // block counts whose thread totals are multiples of pieces_per_row
  const int P = p.pieces_per_row;
  int g = std::__gcd(kThreads, P);
  int unit = P / g;
  long rows = (long)B * T_max;
  long want_threads = std::max<long>(P, std::min<long>(rows * P, 512L * kThreads));
  int want_blocks = (int)((want_threads + kThreads - 1) / kThreads);
  p.amax_blocks = round_to_unit(std::min(want_blocks, 512), unit);
  long enc_threads = std::max<long>(P, std::min<long>(rows * P, 2048L * kThreads));
  int enc_blocks = (int)((enc_threads + kThreads - 1) / kThreads);
  p.encode_blocks = round_to_unit(std::min(enc_blocks, 2048), unit);
  return p;
}

size_t quant_workspace_bytes(const QuantPlan &p) {
  size_t n = (size_t)p.amax_blocks * p.groups * sizeof(uint32_t);
  return (n + 255) & ~(size_t)255;
}

hipError_t launch_kv_quant(const uint16_t *x, wa_strides xs, int B, int H, int T_max,
                           const int32_t *lens, const int32_t *dst_start, uint8_t *cache,
                           wa_strides cs, int cache_len, float *scale, int per_head,
                           int compute_scale, uint32_t *ws, const QuantPlan &plan,
                           hipStream_t stream) {
  (void)H;
  const size_t lds = (size_t)plan.groups * sizeof(uint32_t);
  if (compute_scale) {
    hipLaunchKernelGGL(kv_amax_kernel, dim3(plan.amax_blocks), dim3(kThreads), lds, stream, x,
                       xs, B, T_max, plan.pieces_per_row, lens, per_head, plan.groups, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kv_encode_kernel, dim3(plan.encode_blocks), dim3(kThreads), lds, stream, x,
                     xs, B, T_max, plan.pieces_per_row, lens, dst_start, cache, cs, cache_len,
                     scale, per_head, plan.groups, compute_scale, ws, plan.amax_blocks);
  return hipGetLastError();
}

}  // namespace wa
