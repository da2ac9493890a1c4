// bf16 -> OCP float8 (E4M3, or E5M2) KV-cache quantization for gfx950.
//
// The dynamic per-tensor / per-head scaling of whisper-blaze 0.1.8 (PyPI
// page, "Direct Kernel API": quantise_e4m3 returns codes and a scale; its
// feature list names E4M3 and E5M2) applied to the KV cache that the HF blog
// "Blazingly fast whisper transcriptions with Inference Endpoints" (section
// "Inference Stack") stores in one byte.
//
// Work split.  A row (one token of one sequence) is H*64 bf16 = P pieces of
// 16 bytes; piece p belongs to head p/8.  A block has lcm(64, P) threads when
// that fits in 1024 (320 for 20 heads), so it covers rows_per_pass whole rows
// at once and thread i always owns piece i % P: its head -- its scale group
// -- never changes, and the 8 lanes of one head sit side by side in a wave.
// Block (b, c) handles rows [c*R, (c+1)*R) of sequence b clipped to lens[b]
// (R = rows_per_pass * loads per thread); every load of a thread is issued
// before the first is used.  Wider rows (P > 1024) fall back to 1024 threads
// that loop over pieces.
//
//   kv_amax_kernel      max of (bits & 0x7fff) per thread -- an exact,
//                       order-free integer max equal to the fp32 abs-max of
//                       the bf16 values -- folded over the 8 lanes of a head
//                       (or the whole wave) and in LDS, one partial per block
//                       and group, stored group-major.
//   kv_scale_kernel     one block per group folds that group's partials and
//                       writes scale[g] = amax_g / FMAX (1 when amax_g is 0),
//                       FMAX = 448 (E4M3) or 57344 (E5M2).
//   kv_encode_kernel    divides each value by scale[g] (IEEE fp32 division),
//                       clamps to +-FMAX, converts pairs with the hardware OCP
//                       fp8/bf8 conversion (round to nearest even) and writes
//                       8 code bytes per piece into the cache slot.
#include <algorithm>

#include "fp8_encode.h"
#include "wa_internal.h"

namespace wa {
namespace {

constexpr int kAmaxLoads = 8;    // rows per thread in the amax pass
constexpr int kEncLoads = 4;     // rows per thread in the encode pass

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

__device__ __forceinline__ int seq_len(const int32_t *lens, int b, int T_max) {
  const int n = lens ? lens[b] : T_max;
  return min(max(n, 0), T_max);
}

// The piece and row offset a thread owns, from the block shape in QuantPlan.
struct Lane {
  int piece;      // first piece (of pieces_per_thread, blockDim apart)
  int row;        // row offset inside a pass
  bool active;
};
__device__ __forceinline__ Lane lane_of(int P, int rows_per_pass) {
  Lane l;
  const int tid = threadIdx.x;
  if (rows_per_pass > 0) {   // blockDim is a multiple of P, or P rounded up to waves
    l.piece = tid % P;
    l.row = tid / P;
    l.active = l.row < rows_per_pass;
  } else {                   // P > blockDim: loop over pieces
    l.piece = tid;
    l.row = 0;
    l.active = true;
  }
  return l;
}

// blockIdx.z picks the tensor (K or V of a pair call; 0 for one tensor).
__global__ __launch_bounds__(1024) void kv_amax_kernel(QuantTensors qt, int T_max, int P,
                                                       int rows_per_pass,
                                                       const int32_t *__restrict__ lens,
                                                       int per_head, int groups,
                                                       uint32_t *__restrict__ partial) {
  extern __shared__ uint32_t smax[];  // [groups]
  const int b = blockIdx.x;
  const uint16_t *__restrict__ x = qt.x[blockIdx.z];
  const wa_strides xs = qt.xs[blockIdx.z];
  const int rpp = max(rows_per_pass, 1);
  const int t0 = blockIdx.y * rpp * kAmaxLoads;
  const int t1 = min(t0 + rpp * kAmaxLoads, seq_len(lens, b, T_max));
  const long n_blocks = (long)gridDim.x * gridDim.y;
  const long blk = (long)blockIdx.y * gridDim.x + blockIdx.x;
  for (int g = threadIdx.x; g < groups; g += blockDim.x) smax[g] = 0;
  __syncthreads();
  const Lane ln = lane_of(P, rows_per_pass);
  const int step = rows_per_pass > 0 ? P : (int)blockDim.x;
  for (int p = ln.piece; p < P; p += (rows_per_pass > 0 ? P : step)) {
    const uint16_t *xp = x + (long)b * xs.b + (long)(p >> 3) * xs.h + (p & 7) * 8;
    uint32_t m = 0;
    if (ln.active) {
      uint4 v[kAmaxLoads];
#pragma unroll
      for (int u = 0; u < kAmaxLoads; ++u) {
        const int t = t0 + ln.row + u * rpp;
        v[u] = t < t1 ? *reinterpret_cast<const uint4 *>(xp + (long)t * xs.t) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kAmaxLoads; ++u) m = max(m, maxabs_bits8(v[u]));
    }
    // the 8 lanes of one head are adjacent and 8-aligned (P is a multiple of 8)
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2));
    m = max(m, (uint32_t)__shfl_xor((int)m, 4));
    if ((threadIdx.x & 7) == 0 && ln.active) atomicMax(&smax[per_head ? (p >> 3) : 0], m);
    if (rows_per_pass > 0) break;
  }
  __syncthreads();
  uint32_t *pz = partial + (long)blockIdx.z * groups * n_blocks;
  for (int g = threadIdx.x; g < groups; g += blockDim.x) pz[(long)g * n_blocks + blk] = smax[g];
}

// One block per group (and tensor, blockIdx.z): fold that group's n_blocks
// partials (contiguous).
__global__ __launch_bounds__(256) void kv_scale_kernel(const uint32_t *__restrict__ partial,
                                                       int n_blocks, float fmax, QuantTensors qt) {
  __shared__ uint32_t wmax[4];
  const int g = blockIdx.x;
  float *__restrict__ scale = qt.scale[blockIdx.z];
  const uint32_t *pg = partial + ((long)blockIdx.z * gridDim.x + g) * n_blocks;
  // Every load of a pass is in flight at once: the partials were written on
  // other XCDs, so each read is a full memory round trip (a group of the
  // prompt prefill has 1792 partials: one pass of seven loads per thread).
  uint32_t m = 0;
  for (int j0 = threadIdx.x; j0 < n_blocks; j0 += 256 * 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = j0 + u * 256 < n_blocks ? pg[j0 + u * 256] : 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) m = max(m, v[u]);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t a = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const float amax = __uint_as_float(a << 16);  // bf16 bits -> fp32, exact
    scale[g] = amax == 0.0f ? 1.0f : amax / fmax;
  }
}

template <Fp8 F>
__global__ __launch_bounds__(1024) void kv_encode_kernel(
    QuantTensors qt, int T_max, int P, int rows_per_pass, const int32_t *__restrict__ lens,
    const int32_t *__restrict__ dst_start, wa_strides cs, int cache_len, int per_head) {
  const int b = blockIdx.x;
  const uint16_t *__restrict__ x = qt.x[blockIdx.z];
  const wa_strides xs = qt.xs[blockIdx.z];
  uint8_t *__restrict__ cache = qt.cache[blockIdx.z];
  const float *__restrict__ scale = qt.scale[blockIdx.z];
  const int rpp = max(rows_per_pass, 1);
  const int t0 = blockIdx.y * rpp * kEncLoads;
  const int t1 = min(t0 + rpp * kEncLoads, seq_len(lens, b, T_max));
  if (t0 >= t1) return;
  const int d0 = dst_start ? dst_start[b] : 0;
  // slots outside [0, cache_len) are skipped
  const int ta = max(t0, -d0), tb = min(t1, cache_len - d0);
  const Lane ln = lane_of(P, rows_per_pass);
  if (!ln.active) return;
  for (int p = ln.piece; p < P; p += (rows_per_pass > 0 ? P : (int)blockDim.x)) {
    const int h = p >> 3;
    const float s = scale[per_head ? h : 0];
    const uint16_t *xp = x + (long)b * xs.b + (long)h * xs.h + (p & 7) * 8;
    uint8_t *cp = cache + (long)b * cs.b + (long)h * cs.h + (long)d0 * cs.t + (p & 7) * 8;
    uint4 v[kEncLoads];
#pragma unroll
    for (int u = 0; u < kEncLoads; ++u) {
      const int t = t0 + ln.row + u * rpp;
      if (t >= ta && t < tb) v[u] = *reinterpret_cast<const uint4 *>(xp + (long)t * xs.t);
    }
    if (fast_scale(s)) {
      const float r = 1.0f / s;
#pragma unroll
      for (int u = 0; u < kEncLoads; ++u) {
        const int t = t0 + ln.row + u * rpp;
        if (t >= ta && t < tb) *reinterpret_cast<uint2 *>(cp + (long)t * cs.t) = encode8_fast<F>(v[u], s, r);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kEncLoads; ++u) {
        const int t = t0 + ln.row + u * rpp;
        if (t >= ta && t < tb) *reinterpret_cast<uint2 *>(cp + (long)t * cs.t) = encode8<F>(v[u], s);
      }
    }
    if (rows_per_pass > 0) break;
  }
}

int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

}  // namespace

QuantPlan quant_plan(int B, int H, int T_max, wa_scale_gran gran) {
  QuantPlan p;
  p.pieces_per_row = H * 8;
  p.groups = gran == WA_SCALE_PER_HEAD ? H : 1;
  const int P = p.pieces_per_row;
  const long l = (long)P / gcd_int(P, 64) * 64;   // lcm(64, P)
  if (l <= 1024) {
    p.threads = (int)l;
    p.rows_per_pass = (int)(l / P);
  } else if (P <= 1024) {
    p.threads = ((P + 63) / 64) * 64;
    p.rows_per_pass = 1;
  } else {
    p.threads = 1024;
    p.rows_per_pass = 0;    // threads loop over pieces, one row per pass
  }
  const int rpp = std::max(p.rows_per_pass, 1);
  p.amax_chunks = (T_max + rpp * kAmaxLoads - 1) / (rpp * kAmaxLoads);
  p.enc_chunks = (T_max + rpp * kEncLoads - 1) / (rpp * kEncLoads);
  p.blocks = (long)B * p.amax_chunks;
  return p;
}

size_t quant_workspace_bytes(const QuantPlan &p) {
  const size_t n = (size_t)p.blocks * p.groups * sizeof(uint32_t);
  return (n + 255) & ~(size_t)255;
}

hipError_t launch_kv_quant(const QuantTensors &qt, int n_tensors, int B, int H, int T_max,
                           const int32_t *lens, const int32_t *dst_start, wa_strides cs,
                           int cache_len, int per_head, int compute_scale, Fp8 fmt, uint32_t *ws,
                           const QuantPlan &plan, hipStream_t stream) {
  (void)H;
  if (compute_scale) {
    const size_t lds = (size_t)plan.groups * sizeof(uint32_t);
    hipLaunchKernelGGL(kv_amax_kernel, dim3(B, plan.amax_chunks, n_tensors), dim3(plan.threads), lds,
                       stream, qt, T_max, plan.pieces_per_row, plan.rows_per_pass, lens, per_head,
                       plan.groups, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float fmax = fmt == Fp8::E4M3 ? fp8_max<Fp8::E4M3>() : fp8_max<Fp8::E5M2>();
    hipLaunchKernelGGL(kv_scale_kernel, dim3(plan.groups, 1, n_tensors), dim3(256), 0, stream, ws,
                       (int)plan.blocks, fmax, qt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  auto kernel = fmt == Fp8::E4M3 ? kv_encode_kernel<Fp8::E4M3> : kv_encode_kernel<Fp8::E5M2>;
  hipLaunchKernelGGL(kernel, dim3(B, plan.enc_chunks, n_tensors), dim3(plan.threads), 0, stream, qt,
                     T_max, plan.pieces_per_row, plan.rows_per_pass, lens, dst_start, cs, cache_len,
                     per_head);
  return hipGetLastError();
}

}  // namespace wa
