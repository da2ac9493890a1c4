// Dense bf16 softmax attention for gfx950: Whisper encoder self-attention
// (no mask, 1500 frames per 30-s chunk) and the causal, ragged decoder
// prompt prefill -- the encoder_self_attn / decoder_self_attn pair of
// whisper-blaze 0.1.8 ("Direct Kernel API"), placed in the model as in
// "Unlocking the power of OpenAI's Whisper", section 3.
//
// One block = 4 waves = 128 queries of one (b, h); each wave owns 32 queries
// and walks the keys in tiles of 64 staged through LDS (double buffered).
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
// to bf16 in place, with no shuffles.  V is transposed once per tile while it
// is written to LDS; all LDS tiles use an XOR swizzle of their 16-byte
// chunks so the MFMA operand reads are bank-conflict free.
//
// The softmax is online (running max and sum per query) in the exp2 domain:
// softmax_scale * log2(e) is folded into one FMA per score.
#include <cmath>

#include "wa_internal.h"

namespace wa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;   // queries per block
constexpr int kBN = 64;            // keys per tile
constexpr int kTileBytes = kBN * 64 * 2;
constexpr float kLog2e = 1.4426950408889634f;

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
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

struct TileRegs {
  uint4 k[2];
  uint4 v[2];
};

__device__ __forceinline__ void load_tile(TileRegs &t, const uint16_t *kp, wa_strides ks,
                                          const uint16_t *vp, wa_strides vs, int k0, int kend,
                                          int tid) {
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + i * kThreads;
    const int row = p >> 3, ch = p & 7;
    const int j = k0 + row;
    t.k[i] = j < kend ? *reinterpret_cast<const uint4 *>(kp + (long)j * ks.t + ch * 8)
                      : make_uint4(0, 0, 0, 0);
  }
  const int pair = w * 8 + (lane >> 3), ch = lane & 7;
  const int j = k0 + 2 * pair;
  t.v[0] = j < kend ? *reinterpret_cast<const uint4 *>(vp + (long)j * vs.t + ch * 8)
                    : make_uint4(0, 0, 0, 0);
  t.v[1] = j + 1 < kend ? *reinterpret_cast<const uint4 *>(vp + (long)(j + 1) * vs.t + ch * 8)
                        : make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ void store_tile(const TileRegs &t, uint8_t *kl, uint8_t *vtl, int tid) {
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + i * kThreads;
    const int row = p >> 3, ch = p & 7;
    *reinterpret_cast<uint4 *>(kl + lds_off(row, ch)) = t.k[i];
  }
  // V^T: dims become rows; this thread holds keys 2*pair and 2*pair+1
  const int pair = w * 8 + (lane >> 3), ch = lane & 7;
  const uint32_t a[4] = {t.v[0].x, t.v[0].y, t.v[0].z, t.v[0].w};
  const uint32_t b[4] = {t.v[1].x, t.v[1].y, t.v[1].z, t.v[1].w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t word = (i & 1) ? ((a[i >> 1] >> 16) | (b[i >> 1] & 0xffff0000u))
                                  : ((a[i >> 1] & 0xffffu) | (b[i >> 1] << 16));
    const int d = ch * 8 + i;
    *reinterpret_cast<uint32_t *>(vtl + lds_off(d, pair >> 2) + (pair & 3) * 4) = word;
  }
}

__global__ __launch_bounds__(kThreads, 2) void encoder_attn_kernel(
    const uint16_t *__restrict__ q, wa_strides qs, const uint16_t *__restrict__ k, wa_strides ks,
    const uint16_t *__restrict__ v, wa_strides vs, uint16_t *__restrict__ o, wa_strides os, int H,
    int T_max, const int32_t *__restrict__ lens, int causal, float c_log2, int n_qt, int total) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];

  // XCD-aware order: blocks are dispatched round robin over the 8 XCDs, so
  // block L runs on XCD L % 8.  Give each XCD a contiguous run of work items
  // so the query tiles of one (b, h) share that XCD's L2 copy of K and V.
  const int per = gridDim.x / 8;
  const int item = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (item >= total) return;
  const int bh = item / n_qt;
  int qt = item - bh * n_qt;
  if (causal) qt = n_qt - 1 - qt;  // longest rows first
  const int b = bh / H, h = bh - b * H;
  const int len = min(max(lens ? lens[b] : T_max, 0), T_max);
  const int q0 = qt * kBM;
  if (q0 >= len) return;
  const int kend = causal ? min(len, q0 + kBM) : len;
  const int nt = (kend + kBN - 1) / kBN;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int my_q = q0 + w * 32 + col;

  // Q^T operand: lane holds query my_q, dims c*16 + half*8 .. +8
  bf16x8 qreg[4];
  {
    const uint16_t *qp = q + (long)b * qs.b + (long)my_q * qs.t + (long)h * qs.h + half * 8;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (my_q < len) {
        qreg[c] = *reinterpret_cast<const bf16x8 *>(qp + c * 16);
      } else {
        qreg[c] = bf16x8{};
      }
    }
  }

  const uint16_t *kp = k + (long)b * ks.b + (long)h * ks.h;
  const uint16_t *vp = v + (long)b * vs.b + (long)h * vs.h;

  f32x16 oacc[2];
  oacc[0] = f32x16{};
  oacc[1] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  TileRegs pre;
  load_tile(pre, kp, ks, vp, vs, 0, kend, tid);
  store_tile(pre, lds[0][0], lds[0][1], tid);
  __syncthreads();

  const int wq_lo = q0 + w * 32;  // this wave's first query
  for (int kt = 0; kt < nt; ++kt) {
    const int k0 = kt * kBN;
    if (kt + 1 < nt) load_tile(pre, kp, ks, vp, vs, k0 + kBN, kend, tid);

    const bool skip = causal && k0 > wq_lo + 31;  // every key after every query of this wave
    if (!skip) {
      const uint8_t *kl = lds[kt & 1][0];
      const uint8_t *vtl = lds[kt & 1][1];

      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const int row = kb * 32 + swap_bits23(col);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kl + lds_off(row, c * 2 + half));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c], s[kb], 0, 0, 0);
        }
      }

      // s[kb][r] is the score of query my_q and key k0 + kb*32 + (r/8)*16 + half*8 + r%8
      const bool need_mask = (k0 + kBN > len) || (causal && k0 + kBN - 1 > wq_lo);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + (r >> 3) * 16 + half * 8 + (r & 7);
            const bool ok = key < len && (!causal || key <= my_q);
            s[kb][r] = ok ? s[kb][r] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx * c_log2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float lsum = 0.f;
      bf16x8 pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(fmaf(s[kb][hh * 8 + i], c_log2, -m_new));
            lsum += p[i];
          }
          uint32_t wd[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) wd[i] = pack_bf16x2(p[2 * i], p[2 * i + 1]);
          pb[kb * 2 + hh] = __builtin_bit_cast(bf16x8, make_uint4(wd[0], wd[1], wd[2], wd[3]));
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < 2; ++db) oacc[db] *= alpha;

#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int d = db * 32 + col;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vtl + lds_off(d, c * 2 + half));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], oacc[db], 0, 0, 0);
        }
      }
    }

    if (kt + 1 < nt) store_tile(pre, lds[(kt + 1) & 1][0], lds[(kt + 1) & 1][1], tid);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
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
        val.x = pack_bf16x2(oacc[db][r4 * 4 + 0] * inv, oacc[db][r4 * 4 + 1] * inv);
        val.y = pack_bf16x2(oacc[db][r4 * 4 + 2] * inv, oacc[db][r4 * 4 + 3] * inv);
        *reinterpret_cast<uint2 *>(op + d) = val;
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
  hipLaunchKernelGGL(encoder_attn_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, q, qs,
                     k, ks, v, vs, o, os, H, T_max, lens, causal, softmax_scale * kLog2e, n_qt,
                     (int)total);
  return hipGetLastError();
}

}  // namespace wa
