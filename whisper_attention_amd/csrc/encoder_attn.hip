// Dense bf16 softmax attention for gfx950: Whisper encoder self-attention
// (no mask, 1500 frames per 30-s chunk) and the causal, ragged decoder
// prompt prefill -- the encoder_self_attn / decoder_self_attn pair of
// whisper-blaze 0.1.8 ("Direct Kernel API"), placed in the model as in
// "Unlocking the power of OpenAI's Whisper", section 3.
//
// One block = 4 waves = 256 queries of one (b, h); each wave owns 64 queries
// (two 32-query MFMA blocks, so every K and V fragment read from LDS feeds
// two MFMAs) and walks the keys in tiles of 64.
//
// Both products run on v_mfma_f32_32x32x16_bf16 in transposed form, so the
// accumulator's lane index is the query:
//   S^T (keys x queries) = K  . Q^T   A = K rows from LDS, B = Q^T in registers
//   O^T (dims x queries) += V^T . P^T  A = V^T from LDS,  B = P^T in registers
// A lane then holds one query's scores, so the softmax row max/sum needs only
// a local reduction plus one exchange with lane ^ 32, and the rescale of O^T
// is lane-local.  The K rows fed to the first product are permuted (bits 2
// and 3 of the row index swapped) so that the S^T accumulator registers come
// out already in the B-operand order of the second product: P^T is converted
// to bf16 in place, with no shuffles.
//
// K and V tiles are copied global -> LDS by the asynchronous 16-byte
// global_load_lds instruction (no register staging) into two stages: the copy
// of tile t+1 is issued right after the barrier that opens tile t, so it lands
// while tile t is computed; one barrier per tile.  Both tiles are
// stored row-major with an XOR swizzle of their 16-byte chunks (the swizzle is
// applied by choosing which global chunk each lane fetches, since the LDS
// destination of that instruction is fixed per lane).  The V^T operand is
// read with gfx950's transposing LDS read ds_read_b64_tr_b16: within each 16
// lanes it returns 4 keys x 1 dim per lane from 4 rows x 16 dims.
//
// Softmax: online, in the exp2 domain (softmax_scale * log2(e) folded into one
// FMA per score), with a lazy rescale -- the running max moves only when a
// tile max exceeds it by more than 2^8 -- and row sums taken from the bf16
// weights with v_dot2_f32_bf16 (two weights per instruction).
#include <cmath>

#include "wa_internal.h"

namespace wa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 64;            // queries per wave (two 32-query MFMA blocks)
constexpr int kBM = kWaves * kQW;  // queries per block
constexpr int kBN = 64;            // keys per tile
constexpr int kTileBytes = kBN * 64 * 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;      // lazy-rescale threshold, log2 units

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// 16-byte chunk swizzle of a 128-byte LDS row
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ swz(row)) << 4);
}
// row index m of the 32x32 product -> key of the tile it carries
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // v_cvt_pk_bf16_f32: round to nearest even
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
constexpr int kStages = 2;
// s_waitcnt immediate with vmcnt = 0 and expcnt / lgkmcnt left at their maxima
constexpr int kVmcnt0 = 0x3F70;
constexpr int kStageBytes = 2 * kTileBytes;  // K then V

// Issue the asynchronous copy of one K/V tile (rows k0 .. k0+63) into a
// stage.  Wave w copies K rows and V rows [16w, 16w+16), 8 rows per
// instruction; lane l lands in 16-byte LDS slot l of the instruction's 1 KB
// and fetches the global chunk that the swizzle assigns to that slot.  Rows
// at or past kend are clamped to row kend-1 (finite data; their scores are
// masked to -inf, so they carry zero weight).
__device__ __forceinline__ void issue_tile(uint8_t *stage, const uint16_t *kp, wa_strides ks,
                                           const uint16_t *vp, wa_strides vs, int k0, int kend,
                                           int lane, int w) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = w * 16 + i * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    const int j = min(k0 + row, kend - 1);
    uint8_t *dst = stage + (w * 16 + i * 8) * 128;
    __builtin_amdgcn_global_load_lds(kp + (long)j * ks.t + chunk * 8, dst, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vp + (long)j * vs.t + chunk * 8, dst + kTileBytes, 16, 0, 0);
  }
}

__device__ __forceinline__ float max_with_lane_xor32(float x) {
  // v_permlane32_swap: each lane gets its own value and that of lane ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

// Per-wave state of the online softmax.
struct WaveState {
  bf16x8 qreg[2][4];   // Q^T operands [q block][dim chunk]
  f32x16 oacc[2][2];   // O^T accumulators [d block][q block]
  float m_run[2];      // running max per query, exp2 domain
  float l_run[2];      // running sum over this lane's half of the keys
};

// One 64-key tile of one wave: S^T = K.Q^T, masked online softmax, O^T += V^T.P^T.
template <bool kCausal>
__device__ __forceinline__ void attend_tile(WaveState &st, const uint8_t *kl, int k0, int len,
                                            int wq_lo, float c_log2, int lane) {
  const int half = lane >> 5, col = lane & 31;
  const uint8_t *vl = kl + kTileBytes;

  // S^T = K . Q^T: each K fragment feeds both query blocks
  f32x16 s[2][2];  // [key block][q block]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = kb * 32 + swap_bits23(col);
    bf16x8 ka[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      ka[c] = *reinterpret_cast<const bf16x8 *>(kl + lds_off(row, c * 2 + half));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[kb][qb] = f32x16{};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], st.qreg[qb][c], s[kb][qb], 0, 0, 0);
    }
  }

  // s[kb][qb][r]: query wq_lo + qb*32 + col, key k0 + kb*32 + (r/8)*16 + half*8 + r%8
  const bool tail = k0 + kBN > len;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const bool need_mask = tail || (kCausal && k0 + kBN - 1 > wq_lo + qb * 32);
    if (need_mask) {
      // the key's offset in the tile is a constant per (kb, r): compare it
      // with this lane's limit instead of forming every key index
      const int my_q = wq_lo + qb * 32 + col;
      int lim = len - 1 - k0 - half * 8;
      if (kCausal) lim = min(lim, my_q - k0 - half * 8);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + (r >> 3) * 16 + (r & 7);
          s[kb][qb][r] = off <= lim ? s[kb][qb][r] : -INFINITY;
        }
    }
  }
  float mt[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
    mt[qb] = max_with_lane_xor32(mx) * c_log2;
  }
  // Lazy rescale: keep the running max unless some query's tile max exceeds
  // it by more than kLazy (P then stays below 2^kLazy, which the bf16
  // weights and fp32 sums carry exactly as well).
  if (__builtin_amdgcn_ballot_w64(mt[0] > st.m_run[0] + kLazy || mt[1] > st.m_run[1] + kLazy) != 0) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m_new = fmaxf(st.m_run[qb], mt[qb]);
      const float alpha = __builtin_amdgcn_exp2f(st.m_run[qb] - m_new);
      st.l_run[qb] *= alpha;
      st.oacc[0][qb] *= alpha;
      st.oacc[1][qb] *= alpha;
      st.m_run[qb] = m_new;
    }
  }

  // V^T operands: lane holds dim db*32 + col and keys c*16 + half*8 .. +8,
  // gathered by the transposing read from 4 key rows x 16 dims per 16 lanes
  const int tr_a = lane & 15;
  const int tr_row = half * 8 + (tr_a >> 2);
  const int tr_col = ((lane >> 4) & 1) * 16 + (tr_a & 3) * 4;
  bf16x8 va[2][4];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s16x4 t[2];
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        const int row = c * 16 + th * 4 + tr_row;
        const int cc = db * 32 + tr_col;
        t[th] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(vl + lds_off(row, cc >> 3) + (cc & 7) * 2));
      }
      va[db][c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float mneg = -st.m_run[qb];
    float lsum = 0.f;
    bf16x8 pb[4];  // P^T operands per key chunk
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t wd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][hh * 8 + 2 * i], c_log2, mneg));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][hh * 8 + 2 * i + 1], c_log2, mneg));
          wd[i] = pack_bf16x2(p0, p1);
          // row sum of the bf16 weights actually used by P.V
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[i]), kOnes2, lsum, false);
        }
        pb[kb * 2 + hh] = __builtin_bit_cast(bf16x8, make_uint4(wd[0], wd[1], wd[2], wd[3]));
      }
    st.l_run[qb] += lsum;
    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        st.oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][c], pb[c], st.oacc[db][qb], 0, 0, 0);
  }
}

// Two LDS stages as separate objects: with the loop unrolled by two, every
// access names its stage statically, so the compiler can see that a copy into
// one stage does not touch the other and inserts no wait before reading it.
__shared__ __attribute__((aligned(1024))) uint8_t g_stage0[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage1[kStageBytes];

template <bool kCausal>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const uint16_t *__restrict__ q, wa_strides qs, const uint16_t *__restrict__ k, wa_strides ks,
    const uint16_t *__restrict__ v, wa_strides vs, uint16_t *__restrict__ o, wa_strides os, int H,
    int T_max, const int32_t *__restrict__ lens, float c_log2, int n_qt, int total) {
  // XCD-aware order: blocks are dispatched round robin over the 8 XCDs, so
  // block L runs on XCD L % 8.  Give each XCD a contiguous run of work items
  // so the query tiles of one (b, h) share that XCD's L2 copy of K and V.
  const int per = gridDim.x / 8;
  const int item = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (item >= total) return;
  const int bh = item / n_qt;
  int qt = item - bh * n_qt;
  if (kCausal) qt = n_qt - 1 - qt;  // longest rows first
  const int b = bh / H, h = bh - b * H;
  const int len = min(max(lens ? lens[b] : T_max, 0), T_max);
  const int q0 = qt * kBM;
  if (q0 >= len) return;
  const int kend = kCausal ? min(len, q0 + kBM) : len;
  const int nt = (kend + kBN - 1) / kBN;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int wq_lo = q0 + w * kQW;  // this wave's first query

  const uint16_t *kp = k + (long)b * ks.b + (long)h * ks.h;
  const uint16_t *vp = v + (long)b * vs.b + (long)h * vs.h;
  issue_tile(g_stage0, kp, ks, vp, vs, 0, kend, lane, w);

  WaveState st;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int my_q = wq_lo + qb * 32 + col;
    const uint16_t *qp = q + (long)b * qs.b + (long)my_q * qs.t + (long)h * qs.h + half * 8;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      st.qreg[qb][c] = my_q < len ? *reinterpret_cast<const bf16x8 *>(qp + c * 16) : bf16x8{};
#pragma unroll
    for (int db = 0; db < 2; ++db) st.oacc[db][qb] = f32x16{};
    st.m_run[qb] = -INFINITY;
    st.l_run[qb] = 0.f;
  }

  // causal: a wave whose every query precedes every key of a tile skips it
  for (int kt = 0; kt < nt; kt += 2) {
    // even tile: stage 0; this wave's copies of it are complete (the
    // compiler does not order the asynchronous copies before the barrier by
    // itself), then the barrier: tile kt is in LDS, stage 1 is free
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (kt + 1 < nt) issue_tile(g_stage1, kp, ks, vp, vs, (kt + 1) * kBN, kend, lane, w);
    if (!(kCausal && kt * kBN > wq_lo + kQW - 1))
      attend_tile<kCausal>(st, g_stage0, kt * kBN, len, wq_lo, c_log2, lane);
    if (kt + 1 >= nt) break;
    // odd tile: stage 1
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (kt + 2 < nt) issue_tile(g_stage0, kp, ks, vp, vs, (kt + 2) * kBN, kend, lane, w);
    if (!(kCausal && (kt + 1) * kBN > wq_lo + kQW - 1))
      attend_tile<kCausal>(st, g_stage1, (kt + 1) * kBN, len, wq_lo, c_log2, lane);
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int my_q = wq_lo + qb * 32 + col;
    const float l_tot = st.l_run[qb] + __shfl_xor(st.l_run[qb], 32, 64);
    if (my_q < len) {
      const float inv = 1.0f / l_tot;
      uint16_t *op = o + (long)b * os.b + (long)my_q * os.t + (long)h * os.h;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          // accumulator rows 8*r4 + 4*half + 0..3 are dims db*32 + that
          const int d = db * 32 + 8 * r4 + 4 * half;
          uint2 val;
          val.x = pack_bf16x2(st.oacc[db][qb][r4 * 4 + 0] * inv, st.oacc[db][qb][r4 * 4 + 1] * inv);
          val.y = pack_bf16x2(st.oacc[db][qb][r4 * 4 + 2] * inv, st.oacc[db][qb][r4 * 4 + 3] * inv);
          *reinterpret_cast<uint2 *>(op + d) = val;
        }
    }
  }
}

}  // namespace

hipError_t launch_encoder(const uint16_t *q, wa_strides qs, const uint16_t *k, wa_strides ks,
                          const uint16_t *v, wa_strides vs, uint16_t *o, wa_strides os, int B,
                          int H, int T_max, const int32_t *lens, int causal,
                          float softmax_scale, hipStream_t stream) {
  const int n_qt = (T_max + kBM - 1) / kBM;
  const long total = (long)B * H * n_qt;
  const long grid = (total + 7) / 8 * 8;
  if (causal)
    hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, q,
                       qs, k, ks, v, vs, o, os, H, T_max, lens, softmax_scale * kLog2e, n_qt,
                       (int)total);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, q,
                       qs, k, ks, v, vs, o, os, H, T_max, lens, softmax_scale * kLog2e, n_qt,
                       (int)total);
  return hipGetLastError();
}

}  // namespace wa
