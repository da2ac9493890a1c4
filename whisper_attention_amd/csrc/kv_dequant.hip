// OCP float8 (E4M3 or E5M2) KV cache -> bf16 for gfx950: the dequantise
// step of whisper-blaze 0.1.8 (PyPI page, "Direct Kernel API":
// dequantise_e4m3 takes the codes and the scale that quantise_e4m3 returned;
// the feature list names "FP8 quantize/dequantize with per-tensor scaling").
//
//   x[b][t][h][:] = bf16_rne(fp32(decode(cache[b][h][t][:]) * scale[g]))
//
// Block (c, h, b) covers slots [c*kRows, (c+1)*kRows) of head h of sequence
// b, clipped to the sequence's valid length.  Four lanes share one 64-code
// slot: each loads 16 codes (16 bytes), converts pairs with the hardware OCP
// fp8/bf8 -> fp32 conversion (exact), multiplies by the scale in fp32 and
// stores 16 bf16 (two 16-byte stores, round to nearest even).  A wave reads
// 16 consecutive slots (1 KB of the cache, contiguous) and writes 16 whole
// 128-byte rows of x; both loads of a lane are issued before either is used.
#include "fp8_encode.h"
#include "wa_internal.h"

namespace wa {
namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 2;                        // slots per lane
constexpr int kRowsPerPass = kThreads / 4;       // 64 slots per pass
constexpr int kRows = kRowsPerPass * kLoads;     // 128 slots per block

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Codes in bytes (2*kHi, 2*kHi+1) of w -> two fp32 values, exact.
template <Fp8 F, bool kHi> __device__ __forceinline__ f32x2 decode_pair(uint32_t w) {
  if constexpr (F == Fp8::E4M3) return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHi);
  else return __builtin_amdgcn_cvt_pk_f32_bf8((int)w, kHi);
}

__device__ __forceinline__ uint32_t to_bf16x2(f32x2 v) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 4 codes (one dword, byte i = element i) -> 4 bf16 (element i in half i).
template <Fp8 F> __device__ __forceinline__ uint2 dequant4(uint32_t w, float s) {
  f32x2 lo = decode_pair<F, false>(w), hi = decode_pair<F, true>(w);
  lo.x *= s;
  lo.y *= s;
  hi.x *= s;
  hi.y *= s;
  return make_uint2(to_bf16x2(lo), to_bf16x2(hi));
}

template <Fp8 F>
__global__ __launch_bounds__(kThreads) void kv_dequant_kernel(
    const uint8_t *__restrict__ cache, wa_strides cs, int n_max, const int32_t *__restrict__ lens,
    const float *__restrict__ scale, int per_head, uint16_t *__restrict__ x, wa_strides xs) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int n = lens ? min(max(lens[b], 0), n_max) : n_max;
  const int t0 = blockIdx.x * kRows;
  if (t0 >= n) return;
  const float s = scale[per_head ? h : 0];
  const int quarter = threadIdx.x & 3;
  const int r = threadIdx.x >> 2;
  const uint8_t *cp = cache + (long)b * cs.b + (long)h * cs.h + quarter * 16;
  uint16_t *xp = x + (long)b * xs.b + (long)h * xs.h + quarter * 16;
  uint4 v[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int t = t0 + r + u * kRowsPerPass;
    if (t < n) v[u] = load_stream(cp + (long)t * cs.t);
  }
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int t = t0 + r + u * kRowsPerPass;
    if (t < n) {
      const uint2 a = dequant4<F>(v[u].x, s), c = dequant4<F>(v[u].y, s);
      const uint2 d = dequant4<F>(v[u].z, s), e = dequant4<F>(v[u].w, s);
      uint4 *dst = reinterpret_cast<uint4 *>(xp + (long)t * xs.t);
      dst[0] = make_uint4(a.x, a.y, c.x, c.y);
      dst[1] = make_uint4(d.x, d.y, e.x, e.y);
    }
  }
}

}  // namespace

hipError_t launch_kv_dequant(const uint8_t *cache, wa_strides cs, int cache_len, const float *scale,
                             int per_head, Fp8 fmt, const int32_t *lens, int B, int H, int T_max,
                             uint16_t *x, wa_strides xs, hipStream_t stream) {
  const int n_max = T_max < cache_len ? T_max : cache_len;
  const dim3 grid((n_max + kRows - 1) / kRows, H, B);
  auto kernel = fmt == Fp8::E4M3 ? kv_dequant_kernel<Fp8::E4M3> : kv_dequant_kernel<Fp8::E5M2>;
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, cache, cs, n_max, lens, scale,
                     per_head, x, xs);
  return hipGetLastError();
}

}  // namespace wa
