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
// (R = rows_per_pass * rows per thread).  Wider rows (P > 1024) fall back to
// 1024 threads that loop over pieces.
//
//   kv_amax_kernel      max of (bits & 0x7fff) per thread -- an exact,
//                       order-free integer max equal to the fp32 abs-max of
//                       the bf16 values -- folded over the 8 lanes of a head
//                       (or the whole wave) and in LDS, one partial per block
//                       and group, stored group-major.  Then each block takes
//                       a ticket from a device-scope counter; the block that
//                       draws the last one folds every partial and writes
//                       scale[g] = amax_g / FMAX (1 when amax_g is 0), FMAX =
//                       448 (E4M3) or 57344 (E5M2), and sets the counter back
//                       to zero.  No block waits for another.
//   kv_encode_kernel    divides each value by scale[g] (IEEE fp32 division),
//                       clamps to +-FMAX, converts pairs with the hardware OCP
//                       fp8/bf8 conversion (round to nearest even) and writes
//                       8 code bytes per piece into the cache slot.
#include <algorithm>

#include "fp8_encode.h"
#include "wa_internal.h"

namespace wa {
namespace {

// Shapes measured on the prefill fill (K and V, 128 prompts, 20 heads):
// 64 rows per amax block (two batches of 16 loads per thread) keeps the
// partials few enough that the last block folds a group's 512 of them in one
// batch of loads; 16-row blocks (1792 partials a group) made the fold alone
// take ~30 us.
constexpr int kAmaxBatch = 16;   // loads in flight per thread in the amax pass
constexpr int kAmaxBatches = 2;  // batches per thread
constexpr int kAmaxLoads = kAmaxBatch * kAmaxBatches;
constexpr int kEncLoads = 4;     // rows per thread in the encode pass
constexpr int kFoldBatch = 32;   // partial loads in flight per lane in the fold
constexpr int kTicketWords = 64; // the per-tensor workspace starts with the ticket counter (256 bytes)
// Amax blocks per sequence at most (a longer sequence's blocks stride over
// its row chunks), so that the partials, and the workspace, do not grow with
// the sequence length: 32 chunks of 64 rows cover 2048 positions at 20 heads.
constexpr int kMaxAmaxChunks = 32;

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

// blockIdx.z picks the tensor (K or V of a pair call; 0 for one tensor).  The
// tensor's workspace is ws + z * ws_words: the ticket counter in word 0, the
// partials from word kTicketWords, group-major.
__global__ __launch_bounds__(1024) void kv_amax_kernel(QuantTensors qt, int T_max, int P,
                                                       int rows_per_pass,
                                                       const int32_t *__restrict__ lens,
                                                       int per_head, int groups, uint32_t *ws,
                                                       long ws_words, float fmax) {
  extern __shared__ uint32_t smax[];  // [groups]
  __shared__ int s_last;
  const int b = blockIdx.x;
  const uint16_t *__restrict__ x = qt.x[blockIdx.z];
  const wa_strides xs = qt.xs[blockIdx.z];
  const int rpp = max(rows_per_pass, 1);
  const int rows_blk = rpp * kAmaxLoads;   // rows of one chunk
  const int n_len = seq_len(lens, b, T_max);
  const long n_blocks = (long)gridDim.x * gridDim.y;
  const long blk = (long)blockIdx.y * gridDim.x + blockIdx.x;
  for (int g = threadIdx.x; g < groups; g += blockDim.x) smax[g] = 0;
  __syncthreads();
  const Lane ln = lane_of(P, rows_per_pass);
  const int step = rows_per_pass > 0 ? P : (int)blockDim.x;
  for (int p = ln.piece; p < P; p += (rows_per_pass > 0 ? P : step)) {
    const uint16_t *xp = x + (long)b * xs.b + (long)(p >> 3) * xs.h + (p & 7) * 8;
    uint32_t m = 0;
    // this block's row chunks: blockIdx.y, then every gridDim.y-th
    for (int t0 = blockIdx.y * rows_blk; ln.active && t0 < n_len; t0 += gridDim.y * rows_blk) {
      const int t1 = min(t0 + rows_blk, n_len);
      if (t0 + ln.row >= t1) break;
      // rows past the end re-read the last valid row, which leaves a max
      // unchanged; one batch of loads in flight at a time
#pragma unroll 1
      for (int bt = 0; bt < kAmaxBatches; ++bt) {
        const int tb = t0 + ln.row + bt * kAmaxBatch * rpp;
        if (tb >= t1) break;
        uint4 v[kAmaxBatch];
#pragma unroll
        for (int u = 0; u < kAmaxBatch; ++u) {
          const int t = min(tb + u * rpp, t1 - 1);
          v[u] = *reinterpret_cast<const uint4 *>(xp + (long)t * xs.t);
        }
#pragma unroll
        for (int u = 0; u < kAmaxBatch; ++u) m = max(m, maxabs_bits8(v[u]));
      }
    }
    // the 8 lanes of one head are adjacent and 8-aligned (P is a multiple of 8)
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2));
    m = max(m, (uint32_t)__shfl_xor((int)m, 4));
    if ((threadIdx.x & 7) == 0 && ln.active) atomicMax(&smax[per_head ? (p >> 3) : 0], m);
    if (rows_per_pass > 0) break;
  }
  __syncthreads();
  uint32_t *wz = ws + (long)blockIdx.z * ws_words;
  uint32_t *pz = wz + kTicketWords;
  // Publish the partials, then take a ticket; the block that draws the last
  // one folds them all.  Everything another block reads -- the partials, the
  // counter -- is written and read with agent-scope atomic operations, which
  // the XCDs' L2 caches do not hold back (they are not coherent with each
  // other); each partial store is complete (its vmcnt drained) before this
  // block's barrier and so before its ticket, and the last block reads the
  // partials after its ticket returned.  An agent-scope fence would do the
  // same by writing back and invalidating a whole L2 in every block.
  for (int g = threadIdx.x; g < groups; g += blockDim.x)
    __hip_atomic_store(&pz[(long)g * n_blocks + blk], smax[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(wz, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(n_blocks - 1);
  __syncthreads();
  if (!s_last) return;
  // lanes per group: the largest power of two, at most a wave, that gives
  // every group a slice of its own when the block is wide enough
  int L = 64;
  while (L > 1 && L * groups > (int)blockDim.x) L >>= 1;
  const int li = threadIdx.x % L;
  float *__restrict__ scale = qt.scale[blockIdx.z];
  const int n = (int)n_blocks;
  for (int g = threadIdx.x / L; g < groups; g += blockDim.x / L) {
    const uint32_t *pg = pz + (long)g * n_blocks;
    uint32_t mg = 0;
    for (int i0 = li; i0 < n; i0 += L * kFoldBatch) {
      uint32_t v[kFoldBatch];
#pragma unroll
      for (int u = 0; u < kFoldBatch; ++u)
        v[u] = __hip_atomic_load(&pg[min(i0 + u * L, n - 1)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int u = 0; u < kFoldBatch; ++u) mg = max(mg, v[u]);
    }
    for (int o = 1; o < L; o <<= 1) mg = max(mg, (uint32_t)__shfl_xor((int)mg, o, L));
    if (li == 0) {
      const float amax = __uint_as_float(mg << 16);  // bf16 bits -> fp32, exact
      scale[g] = amax == 0.0f ? 1.0f : amax / fmax;
    }
  }
  // every ticket of this call is drawn: the next call starts from zero
  if (threadIdx.x == 0) __hip_atomic_store(wz, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// kDyn: the scales were just computed from these values (no element exceeds
// its group's amax), so the reciprocal quotient needs no clamp.
template <Fp8 F, bool kDyn>
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
        if (t >= ta && t < tb)
          *reinterpret_cast<uint2 *>(cp + (long)t * cs.t) =
              kDyn ? encode8_dyn<F>(v[u], s, r) : encode8_fast<F>(v[u], s, r);
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
  p.amax_chunks = std::min((T_max + rpp * kAmaxLoads - 1) / (rpp * kAmaxLoads), kMaxAmaxChunks);
  p.enc_chunks = (T_max + rpp * kEncLoads - 1) / (rpp * kEncLoads);
  p.blocks = (long)B * p.amax_chunks;
  return p;
}

size_t quant_workspace_bytes(int B, int groups) {
  const size_t n = kTicketWords * sizeof(uint32_t) + (size_t)B * kMaxAmaxChunks * groups * sizeof(uint32_t);
  return (n + 255) & ~(size_t)255;
}

hipError_t launch_kv_quant(const QuantTensors &qt, int n_tensors, int B, int H, int T_max,
                           const int32_t *lens, const int32_t *dst_start, wa_strides cs,
                           int cache_len, int per_head, int compute_scale, Fp8 fmt, uint32_t *ws,
                           const QuantPlan &plan, hipStream_t stream) {
  (void)H;
  if (compute_scale) {
    const size_t lds = (size_t)plan.groups * sizeof(uint32_t);
    const float fmax = fmt == Fp8::E4M3 ? fp8_max<Fp8::E4M3>() : fp8_max<Fp8::E5M2>();
    hipLaunchKernelGGL(kv_amax_kernel, dim3(B, plan.amax_chunks, n_tensors), dim3(plan.threads), lds,
                       stream, qt, T_max, plan.pieces_per_row, plan.rows_per_pass, lens, per_head,
                       plan.groups, ws, (long)(quant_workspace_bytes(B, plan.groups) / sizeof(uint32_t)), fmax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  auto kernel = fmt == Fp8::E4M3
                    ? (compute_scale ? kv_encode_kernel<Fp8::E4M3, true> : kv_encode_kernel<Fp8::E4M3, false>)
                    : (compute_scale ? kv_encode_kernel<Fp8::E5M2, true> : kv_encode_kernel<Fp8::E5M2, false>);
  hipLaunchKernelGGL(kernel, dim3(B, plan.enc_chunks, n_tensors), dim3(plan.threads), 0, stream, qt,
                     T_max, plan.pieces_per_row, plan.rows_per_pass, lens, dst_start, cs, cache_len,
                     per_head);
  return hipGetLastError();
}

}  // namespace wa
