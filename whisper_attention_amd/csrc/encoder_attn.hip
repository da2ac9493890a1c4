// Dense bf16 softmax attention for gfx950: Whisper encoder self-attention
// (no mask, 1500 frames per 30-s chunk) and the causal, ragged decoder
// prompt prefill -- the encoder_self_attn / decoder_self_attn pair of
// whisper-blaze 0.1.8 ("Direct Kernel API"), placed in the model as in
// "Unlocking the power of OpenAI's Whisper", section 3.
//
// One block = 4 waves = 128 queries of one (b, h); each wave owns one
// 32-query MFMA column block and walks the keys in tiles of 64.  A wave takes
// at most 128 VGPRs and a block 40 KB of LDS, so four blocks share a CU (one
// wave of each on every SIMD): while one wave's matrix work runs, the others'
// vector work and waits fill the SIMD.  (64 queries per wave, two column
// blocks per K and V fragment read, needs 216 VGPRs and so allows two blocks
// per CU: no faster on the 30-s encoder, 5 % slower on the 15-s window, 22 %
// on the 10-s window and 14 % on the prompt prefill.)  A non-causal query
// range of 129 to 256 rows (a prompt attending to the encoder frames) takes
// one block of eight waves per (b, h) instead, so that K and V are copied
// from memory once rather than by two blocks that drift apart and miss in
// L2.
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
// Each interval (one per key tile t) runs the matrix work -- P(t-1).V(t-1)
// and S(t) = K(t).Q^T -- and then the softmax of tile t on the vector ALU.
// Eight waves in two groups that alternate those phases under a shared
// barrier were measured slower than independent four-wave blocks per CU.
//
// K and V tiles are copied global -> LDS by the asynchronous 16-byte
// global_load_lds instruction (no register staging) into two rings, K tile j
// in K slot j % 2 and V tile j in V slot j % 3 (16 + 24 KB): interval t reads
// K of tile t and V of tile t-1 and starts the copy of tile t+1 into the
// slots whose last reads were in interval t-1, so every copy has one
// interval to land; completion is waited for explicitly (vmcnt) before the
// barrier that publishes a tile.  The interval loop is unrolled by six so
// every LDS read names its slot with a constant offset.  Tiles are stored
// row-major with an XOR swizzle of their 16-byte chunks (applied by choosing
// which global chunk each lane fetches, since the LDS destination of that
// instruction is fixed per lane).  The V^T operand is
// read with gfx950's transposing LDS read ds_read_b64_tr_b16: within each 16
// lanes it returns 4 keys x 1 dim per lane from 4 rows x 16 dims.
//
// Softmax: online, in the exp2 domain (softmax_scale * log2(e) folded into one
// FMA per score), against a running reference that is not the exact max: a
// tile's weights are taken against it first, and only a weight of 2 or more
// sends the tile through the exact max and a rescale (new_max below), so the
// common tile spends no vector work on its max.  Row sums of the bf16 weights
// are taken on the matrix pipe by a small 16x16x32 MFMA per key chunk.
//
// fp8 Q and K (kFp8, the aggressive-fp8 variant): E4M3 codes with
// dequantization scales.  K tiles are 4 KB (64-byte rows) and S^T comes from
// one v_mfma_f32_32x32x64_f8f6f4 per 32 x 32 block; the scales join the
// exp2-domain multiplier, and everything after the scores is unchanged.
#include <cmath>

#include "wa_internal.h"

namespace wa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Waves per block: 4 (128 queries), or 8 (256 queries) for a short
// non-causal query range, whose one block per (b, h) then reads K and V once.
template <int kW> constexpr int kCopiesOf = 8 / kW;  // 8-row copies per wave per K/V tile
constexpr int kNQ = 1;                    // 32-query MFMA column blocks per wave
constexpr int kQW = 32 * kNQ;             // queries per wave
template <int kW> constexpr int kBMOf = kW * kQW;   // queries per block
constexpr int kMaxCopies = 2;
constexpr int kBN = 64;                   // keys per tile
constexpr int kTileBytes = kBN * 64 * 2;  // one 64 x 64 bf16 tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kHeadroom = 8.0f;         // running max above the tile max, log2 units
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8): wait until at most N vector-memory operations of
// this wave are outstanding and all its LDS operations are complete.
constexpr int kVmcnt0Lgkm0 = 0x0070;

// 16-byte chunk swizzle of a 128-byte LDS row: the chunk index is XORed with
// bits 1, 2, 3 of the row, reversed.  The K operand reads (16 rows, one chunk)
// and the transposing V reads (rows r..r+3 and r+8..r+11, four chunks) then
// hit distinct banks, and rows 16 apart share a swizzle, so stepping by 16 or
// 32 rows is a constant offset.
__device__ __forceinline__ int swz(int row) {
  return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
}
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ swz(row)) << 4);
}
// row index m of the 32x32 product -> key of the tile it carries
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // v_cvt_pk_bf16_f32: round to nearest even
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float max_with_lane_xor32(float x) {
  // v_permlane32_swap: each lane gets its own value and that of lane ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

// Per-lane byte offsets of the K (and V) row this lane copies in every
// tile, relative to the tile's first row: one copy instruction fills rows
// [row0, row0+8); lane l lands in 16-byte LDS slot l of the instruction's
// 1 KB and fetches the global chunk the swizzle assigns to that slot.  Rows
// at or past kend are clamped to row kend-1 (finite data; their scores are
// masked to -inf, so they carry zero weight).
struct CopyOffsets {
  uint32_t k, v;
};

__device__ __forceinline__ CopyOffsets copy_offsets(wa_strides ks, wa_strides vs, int max_row,
                                                    int lane, int row0) {
  const int row = row0 + (lane >> 3);
  const int chunk = (lane & 7) ^ swz(row);
  const int r = min(row, max_row);
  return CopyOffsets{(uint32_t)((r * ks.t + chunk * 8) * 2), (uint32_t)((r * vs.t + chunk * 8) * 2)};
}

// fp8 K tiles: 64-byte rows, four 16-byte chunks, chunk index XORed with
// bits 2 and 3 of the row.  The 16 lanes of a K operand read (rows 0..15 in
// the permuted order, one chunk) then cover all 16 slots of 256 bytes.
__device__ __forceinline__ int swz8(int row) { return ((row >> 2) & 1) | (((row >> 3) & 1) << 1); }
__device__ __forceinline__ int lds_off8(int row, int chunk) { return row * 64 + ((chunk ^ swz8(row)) << 4); }

// Per-lane byte offset of the fp8 K row this lane copies: one copy
// instruction fills rows [row0, row0+16), lane l landing in 16-byte LDS slot
// l; rows at or past kend are clamped to row kend-1.
__device__ __forceinline__ uint32_t copy_offset_k8(wa_strides ks, int max_row, int lane, int row0) {
  const int row = row0 + (lane >> 2);
  const int chunk = (lane & 3) ^ swz8(row);
  return (uint32_t)(min(row, max_row) * ks.t + chunk * 16);
}

// The LDS rings: two slots of one K tile and three of one V tile (an fp8 K
// tile uses the first half of its slot).
__shared__ __attribute__((aligned(1024))) uint8_t g_kring[2][kTileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_vring[3][kTileBytes];
// The second key group's rings (two-group blocks only): K slots 0-1, then V
// slots 0-2, in one array so that after the loop the 40 KB also carry the
// group's partial results to the first group.
__shared__ __attribute__((aligned(1024))) uint8_t g_ring1[5][kTileBytes];

// One asynchronous 16-byte-per-lane copy global -> LDS: lane l's 16 bytes,
// read from base + voff, land at LDS byte address lds + 16*l.  Written out
// (rather than with the compiler's global_load_lds builtin) because the
// compiler cannot tell the slots apart across the interval's branches and
// would wait for every copy in flight -- including the next tile's -- before
// each LDS read.  The instruction has no result register; completion
// is tracked explicitly with s_waitcnt vmcnt before the barrier that
// publishes a tile.
__device__ __forceinline__ void copy16_to_lds(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// LDS byte addresses of a K or V slot, as the instruction's M0 wants them.
__device__ __forceinline__ uint32_t k_addr(int slot, bool g1) {
  const uint8_t *base = g1 ? &g_ring1[0][0] : &g_kring[0][0];
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)base + slot * kTileBytes;
}
__device__ __forceinline__ uint32_t v_addr(int slot, bool g1) {
  const uint8_t *base = g1 ? &g_ring1[2][0] : &g_vring[0][0];
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)base + slot * kTileBytes;
}

// Issue the asynchronous copy of the K/V tile that starts at row k0 into K
// slot kslot and V slot vslot.  Wave w of kW fills K rows and V rows
// [w*64/kW, (w+1)*64/kW) of the slots, 8 rows per copy instruction.
// With fp8 K (kFp8) the K tile is 4 KB: waves 0..3 make one 16-row copy each,
// rows [16w, 16w+16), from byte offsets k8 (the full-tile offset) of a uint8 K.
template <bool kFp8, int kW>
__device__ __forceinline__ void issue_tile(int kslot, int vslot, const void *kp, wa_strides ks,
                                           const uint16_t *vp, wa_strides vs, int k0, int kend,
                                           const CopyOffsets (&full)[kMaxCopies], uint32_t k8, int lane,
                                           int w, bool g1) {
  constexpr int kC = kCopiesOf<kW>;
#pragma unroll
  for (int i = 0; i < kC; ++i) {
    const int row0 = (w * kC + i) * 8;
    // only the last tile can run past kend
    const CopyOffsets c = k0 + kBN <= kend ? full[i] : copy_offsets(ks, vs, kend - 1 - k0, lane, row0);
    const uint32_t dst = k_addr(kslot, g1) + row0 * 128;
    if (!kFp8) copy16_to_lds(static_cast<const uint16_t *>(kp) + (long)k0 * ks.t, c.k, dst);
    copy16_to_lds(vp + (long)k0 * vs.t, c.v, v_addr(vslot, g1) + row0 * 128);
  }
  if (kFp8 && w < 4) {  // four 16-row copies fill a 4 KB fp8 K tile
    const int row0 = w * 16;
    const uint32_t off = k0 + kBN <= kend ? k8 : copy_offset_k8(ks, kend - 1 - k0, lane, row0);
    copy16_to_lds(static_cast<const uint8_t *>(kp) + (long)k0 * ks.t, off, k_addr(kslot, g1) + row0 * 64);
  }
}

// Per-wave state of the online softmax.
struct WaveState {
  bf16x8 qreg[kNQ][4];   // Q^T operands [q block][dim chunk]
  f32x16 oacc[2][kNQ];   // O^T accumulators [d block][q block]
  f32x4 lacc[kNQ];       // row sums of P per q block (16x16 MFMA layout, see row_sum_selector)
  float m_run[kNQ];      // running max per query, exp2 domain
  bf16x8 sel;           // 0/1 selector A operand of the row-sum MFMA
};

// Per-lane LDS byte offsets of the operand reads (the same in every tile).
struct ReadOffsets {
  int k[4];    // K rows for MFMA c (key block 0; key block 1 is +4096)
  int k8[2];   // fp8 K: the lane's two 16-byte chunks (key block 1 is +2048)
  int v[2][2]; // V^T transposing reads for (db, th); key chunk c is +2048*c
};

__device__ __forceinline__ ReadOffsets read_offsets(int lane) {
  const int half = lane >> 5, col = lane & 31;
  ReadOffsets r;
  const int krow = swap_bits23(col);
#pragma unroll
  for (int c = 0; c < 4; ++c) r.k[c] = lds_off(krow, c * 2 + half);
  // fp8: operand byte b of lane group `half` is dim 32*half + b
  r.k8[0] = lds_off8(krow, 2 * half);
  r.k8[1] = lds_off8(krow, 2 * half + 1);
  // transposing read: source lane a = lane & 15 points at key row
  // c*16 + th*4 + half*8 + a/4 and dims db*32 + ((lane>>4)&1)*16 + (a%4)*4
  const int a = lane & 15;
  const int row = half * 8 + (a >> 2);
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      const int cc = db * 32 + ((lane >> 4) & 1) * 16 + (a & 3) * 4;
      r.v[db][th] = lds_off(row + th * 4, cc >> 3) + (cc & 7) * 2;
    }
  return r;
}

// S^T = K . Q^T for one key tile: each K fragment feeds both query blocks.
// s[kb][qb][r] is the score of query (qb*32 + col) and key
// kb*32 + (r/8)*16 + half*8 + r%8 of the tile.
template <bool kFp8>
__device__ __forceinline__ void scores(const WaveState &st, const uint8_t *kl,
                                       const ReadOffsets &ro, f32x16 (&s)[2][kNQ]) {
  if (kFp8) {
    // v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3): the whole head dim in one
    // instruction; lane l gives K row l%32 and Q column l%32, dims
    // 32*(l/32) .. +32 in byte order
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint4 a0 = *reinterpret_cast<const uint4 *>(kl + ro.k8[0] + kb * 2048);
      const uint4 a1 = *reinterpret_cast<const uint4 *>(kl + ro.k8[1] + kb * 2048);
      const i32x8 ka = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
      for (int qb = 0; qb < kNQ; ++qb) {
        const uint4 b0 = __builtin_bit_cast(uint4, st.qreg[qb][0]);
        const uint4 b1 = __builtin_bit_cast(uint4, st.qreg[qb][1]);
        const i32x8 qv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        s[kb][qb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qv, f32x16{}, 0, 0, 0, 0, 0, 0);
      }
    }
    return;
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    bf16x8 ka[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      ka[c] = *reinterpret_cast<const bf16x8 *>(kl + ro.k[c] + kb * 4096);
#pragma unroll
    for (int qb = 0; qb < kNQ; ++qb) {
      s[kb][qb] = f32x16{};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], st.qreg[qb][c], s[kb][qb], 0, 0, 0);
    }
  }
}

// P = exp2(S*c - m) for one tile, as bf16 P^T operands.
__device__ __forceinline__ void softmax_exp(const f32x16 (&s)[2][kNQ], const float (&m)[kNQ],
                                            float c_log2, bf16x8 (&pb)[kNQ][4]) {
#pragma unroll
  for (int qb = 0; qb < kNQ; ++qb) {
    const float mneg = -m[qb];
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
        }
        pb[qb][kb * 2 + hh] = __builtin_bit_cast(bf16x8, make_uint4(wd[0], wd[1], wd[2], wd[3]));
      }
  }
}

// Scores of keys at or past the key length, and (causal) of keys after the
// query, to -inf.  Only the last tile and the causal diagonal tiles have any.
template <bool kCausal>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2][kNQ], int k0, int len, int wq_lo, int lane) {
  const int half = lane >> 5, col = lane & 31;
  if (k0 + kBN > len || (kCausal && k0 + kBN - 1 > wq_lo)) {
#pragma unroll
    for (int qb = 0; qb < kNQ; ++qb) {
      // the key's offset in the tile is a constant per (kb, r): compare it
      // with this lane's limit instead of forming every key index
      int lim = len - 1 - k0 - half * 8;
      if (kCausal) lim = min(lim, wq_lo + qb * 32 + col - k0 - half * 8);
      asm volatile("" : "+v"(lim));  // keep the compares inside this branch
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + (r >> 3) * 16 + (r & 7);
          s[kb][qb][r] = off <= lim ? s[kb][qb][r] : -INFINITY;
        }
    }
  }
}

// The running max (exp2 domain) is a reference point, not the exact max:
// softmax is unchanged by a common shift of a row's scores, and the fp32 / bf16
// weights and sums carry any shift that keeps the largest weight well inside
// their range.  Each tile's weights are therefore first taken against the
// running max as it stands; only when one of them reaches 2 (or is not
// finite) is the tile redone: its exact max is taken, the running max moves
// to kHeadroom above it, and O and the row sums are rescaled.  Afterwards the
// tile's largest weight is 2^-kHeadroom, so the reference stays put until a
// score exceeds the max seen so far by more than kHeadroom + 1.
//
// Tile max of the (masked) scores; moves the running max of each query to
// kHeadroom above it when that is higher, and returns in alpha[qb] the factor
// that takes O and l from the old frame to the new one (0 on the first tile,
// 1 where the max stays).
__device__ __forceinline__ void new_max(WaveState &st, const f32x16 (&s)[2][kNQ], float c_log2,
                                        float (&alpha)[kNQ]) {
#pragma unroll
  for (int qb = 0; qb < kNQ; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
    const float mt = max_with_lane_xor32(mx) * c_log2 + kHeadroom;
    const float m_new = fmaxf(st.m_run[qb], mt);
    alpha[qb] = __builtin_amdgcn_exp2f(st.m_run[qb] - m_new);
    st.m_run[qb] = m_new;
  }
}

// Whether any weight of the tile, as packed bf16 P^T operands, is 2 or more,
// inf or NaN: the top exponent bit of a non-negative bf16 is set exactly then.
__device__ __forceinline__ bool weight_reaches_two(const bf16x8 (&pb)[kNQ][4]) {
  uint32_t acc = 0;
#pragma unroll
  for (int qb = 0; qb < kNQ; ++qb)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 u = __builtin_bit_cast(uint4, pb[qb][c]);
      acc |= u.x | u.y | u.z | u.w;
    }
  return __builtin_amdgcn_ballot_w64((acc & 0x40004000u) != 0) != 0;
}

// O and the row sums from the old frame to the new one (after a tile max
// moved the running max).
__device__ __forceinline__ void rescale(WaveState &st, const float (&alpha)[kNQ], int lane) {
#pragma unroll
  for (int qb = 0; qb < kNQ; ++qb) {
    st.oacc[0][qb] *= alpha[qb];
    st.oacc[1][qb] *= alpha[qb];
    // row sums: lane n < 16 holds query n in element 0 and query n+16 in
    // element 1 (see row_sum_selector); the latter's factor is in lane n+16
    const float alpha_hi = __shfl(alpha[qb], (lane & 15) + 16, 64);
    st.lacc[qb][0] *= alpha[qb];
    st.lacc[qb][1] *= alpha_hi;
  }
}

// Row sums of P on the matrix pipe, in the matrix phase: the 16x16x32 MFMA
// with B = a P^T operand (lane l: query l%32, 8 keys of half l/32) and A = a
// 0/1 selector gives D[0][n] = the sum over the chunk's keys for query n and
// D[1][n] = the same for query n+16 (lane n, elements 0 and 1).  This keeps
// the sums off the vector ALU, and v_dot2_f32_bf16, which would halve the
// vector work, does not overlap with MFMA on gfx950: it would stall the other
// group's matrix phase.
__device__ __forceinline__ bf16x8 row_sum_selector(int lane) {
  // A operand of the 16x16x32 MFMA: lane l holds row m = l%16 and 8 values of
  // k-group g = l/16.  Row 0 sums groups 0 and 2 (query n), row 1 groups 1, 3.
  const int m = lane & 15, g = lane >> 4;
  const bool one = (m == 0 && (g & 1) == 0) || (m == 1 && (g & 1) == 1);
  const __bf16 v = (__bf16)(one ? 1.0f : 0.0f);
  return bf16x8{v, v, v, v, v, v, v, v};
}

// O^T += V^T . P^T for one tile.  V^T operands: lane holds dim db*32 + col and
// keys c*16 + half*8 .. +8, gathered by the transposing read.
__device__ __forceinline__ void accumulate_pv(WaveState &st, const uint8_t *vl,
                                              const ReadOffsets &ro, const bf16x8 (&pb)[kNQ][4]) {
#pragma unroll
  for (int qb = 0; qb < kNQ; ++qb)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      st.lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(st.sel, pb[qb][c], st.lacc[qb], 0, 0, 0);
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    bf16x8 va[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vl + ro.v[db][0] + c * 2048));
      const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vl + ro.v[db][1] + c * 2048));
      va[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int qb = 0; qb < kNQ; ++qb)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        st.oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c], pb[qb][c], st.oacc[db][qb], 0, 0, 0);
  }
}

struct Ctx {
  const void *kp;
  const uint16_t *vp;
  wa_strides ks, vs;
  CopyOffsets co[kMaxCopies];
  uint32_t k8;     // fp8 K: this lane's copy offset within a full tile
  ReadOffsets ro;
  int nt, kend, len, wq_lo, lane, w;
  float c_log2;
  bool g1;     // the block's second key group (two-group blocks), else false
};

// Interval t: K of tile t is in `cur`, V of tile t-1 in `prev`; tile t+1 is
// copied into K slot `kahead` (that of tile t-1) and V slot `vahead` (that of
// tile t-2), whose last reads were in interval t-1.  The block's waves pass
// one barrier per interval.
template <bool kFp8, int kW>
__device__ __forceinline__ void open_interval(int kahead, int vahead, int t, const Ctx &x) {
  // Keep every instruction of the previous interval above the barrier.
  __builtin_amdgcn_sched_barrier(0);
  // This wave's copies of tile t are complete (nothing else is in flight),
  // and so are its LDS reads of interval t-1.  Then a bare barrier:
  // afterwards tile t is in LDS for everyone, and the slots read in interval
  // t-1 are free for tile t+1.
  __builtin_amdgcn_s_waitcnt(kVmcnt0Lgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  if (t + 1 < x.nt)
    issue_tile<kFp8, kW>(kahead, vahead, x.kp, x.ks, x.vp, x.vs, (t + 1) * kBN, x.kend, x.co, x.k8, x.lane, x.w,
                         x.g1);
}

// causal: a wave whose every query precedes every key of tile j skips it
template <bool kCausal>
__device__ __forceinline__ bool wave_needs(int j, const Ctx &x) {
  return j >= 0 && j < x.nt && !(kCausal && j * kBN > x.wq_lo + kQW - 1);
}

// Interval t: P(t-1).V(t-1) and S(t) on the matrix cores, then the softmax
// of tile t on the vector ALU (the other block on the CU fills the matrix
// cores meanwhile).  P(t) is carried to the next interval in `pa`.
template <bool kCausal, bool kFp8, int kW>
__device__ __forceinline__ void interval(WaveState &st, bf16x8 (&pa)[kNQ][4], const uint8_t *cur,
                                         const uint8_t *prev, int kahead, int vahead, int t, const Ctx &x) {
  open_interval<kFp8, kW>(kahead, vahead, t, x);
  if (wave_needs<kCausal>(t - 1, x)) accumulate_pv(st, prev, x.ro, pa);
  if (wave_needs<kCausal>(t, x)) {
    f32x16 s[2][kNQ];
    // tile 0 is the first of every wave: it sets the running max
    bool redo = t == 0;
    if (!redo) {
      scores<kFp8>(st, cur, x.ro, s);
      __builtin_amdgcn_sched_barrier(0);  // matrix phase, then vector phase
      mask_tile<kCausal>(s, t * kBN, x.len, x.wq_lo, x.lane);
      softmax_exp(s, st.m_run, x.c_log2, pa);
      // An exponential costs two to four times the issue time of an FMA; the
      // scheduling groups interleave them with the FMAs and conversions,
      // which then issue in their shadow instead of before them.
#pragma unroll
      for (int g = 0; g < 32 * kNQ; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);  // one exponential
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two other vector ops
      }
      redo = weight_reaches_two(pa);
    }
    if (redo) {
      // The scores are read again from LDS (tile t's K slot is not reused
      // before the next interval) rather than kept: the weights overwrite
      // them in place.  The opaque offsets keep the compiler from reusing
      // the first reads.
      ReadOffsets ro = x.ro;
#pragma unroll
      for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(ro.k[c]));
      asm volatile("" : "+v"(ro.k8[0]), "+v"(ro.k8[1]));
      scores<kFp8>(st, cur, ro, s);
      mask_tile<kCausal>(s, t * kBN, x.len, x.wq_lo, x.lane);
      float alpha[kNQ];
      new_max(st, s, x.c_log2, alpha);
      rescale(st, alpha, x.lane);
      softmax_exp(s, st.m_run, x.c_log2, pa);
    }
  }
}

// Rows i < len_q of o for a sequence with no key: the empty sum is zero.
template <int kW>
__device__ __forceinline__ void zero_rows(uint16_t *o, wa_strides os, int b, int h, int q0, int len_q) {
  const int i = q0 + (int)threadIdx.x;
  if ((int)threadIdx.x >= kBMOf<kW> || i >= len_q) return;
  uint4 *op = reinterpret_cast<uint4 *>(o + (long)b * os.b + (long)i * os.t + (long)h * os.h);
#pragma unroll
  for (int c = 0; c < 8; ++c) op[c] = uint4{0u, 0u, 0u, 0u};
}

// kFp8: q and k hold E4M3 codes (uint8, strides in bytes) with
// dequantization scales q_scale / k_scale ([1], or [H] when per_head).
// Queries i < q_lens[b] (of Tq_max rows) attend keys j < k_lens[b] (of Tk_max
// rows); the causal form needs both to be the same sequence.
//
// kG = 2 (non-causal, for grids too small to fill the GPU): the block holds
// two groups of kW waves over the same queries.  The first takes the first
// ceil(n/2) key tiles, the second the rest, each with its own rings, under
// the one barrier per interval; at the end the second group hands its
// running max, row sums and unnormalized O to the first through LDS, which
// combines the two as the split-key merge does (each weighted by 2 to the
// power of its max less the larger max) and writes the output.
template <bool kCausal, bool kFp8, int kW, int kG>
__global__ __launch_bounds__(kW * kG * 64) __attribute__((amdgpu_waves_per_eu(4))) void attn_fwd_kernel(
    const void *__restrict__ q, wa_strides qs, const void *__restrict__ k, wa_strides ks,
    const uint16_t *__restrict__ v, wa_strides vs, uint16_t *__restrict__ o, wa_strides os, int H,
    int Tq_max, const int32_t *__restrict__ q_lens, int Tk_max, const int32_t *__restrict__ k_lens,
    float c_log2, const float *__restrict__ q_scale, const float *__restrict__ k_scale, int per_head,
    int n_qt, int total) {
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
  const int len = min(max(q_lens ? q_lens[b] : Tq_max, 0), Tq_max);
  constexpr int kBM = kBMOf<kW>;
  const int q0 = qt * kBM;
  if (q0 >= len) return;
  const int len_k = min(max(k_lens ? k_lens[b] : Tk_max, 0), Tk_max);
  if (len_k == 0) {
    zero_rows<kW>(o, os, b, h, q0, len);
    return;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave within its key group (read as a scalar: the group is wave-uniform)
  const int wv = kG == 1 ? tid >> 6 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = kG == 1 ? wv : wv % kW;
  const int half = lane >> 5, col = lane & 31;
  Ctx x;
  x.g1 = kG == 2 && wv >= kW;
  // this group's keys: [k_lo, k_lo + len_g)
  int k_lo = 0, len_g = len_k, n0 = 0;
  if (kG == 2) {
    n0 = ((len_k + kBN - 1) / kBN + 1) / 2;
    k_lo = x.g1 ? n0 * kBN : 0;
    len_g = x.g1 ? max(len_k - n0 * kBN, 0) : min(len_k, n0 * kBN);
  }
  x.kp = kFp8 ? (const void *)(static_cast<const uint8_t *>(k) + (long)b * ks.b + (long)h * ks.h +
                               (long)k_lo * ks.t)
              : (const void *)(static_cast<const uint16_t *>(k) + (long)b * ks.b + (long)h * ks.h +
                               (long)k_lo * ks.t);
  x.vp = v + (long)b * vs.b + (long)h * vs.h + (long)k_lo * vs.t;
  x.ks = ks;
  x.vs = vs;
  x.kend = kCausal ? min(len_k, q0 + kBM) : len_g;
  x.nt = (x.kend + kBN - 1) / kBN;
  x.len = len_g;
  // intervals 0 .. nloop: both groups pass the same barriers
  const int nloop = kG == 1 ? x.nt : n0;
  x.wq_lo = q0 + w * kQW;
  x.lane = lane;
  x.w = w;
  // fp8: the scores come out in code units; fold both scales into the
  // exp2-domain multiplier
  x.c_log2 = kFp8 ? c_log2 * q_scale[per_head ? h : 0] * k_scale[per_head ? h : 0] : c_log2;
#pragma unroll
  for (int i = 0; i < kCopiesOf<kW>; ++i)
    x.co[i] = copy_offsets(ks, vs, kBN - 1, lane, (w * kCopiesOf<kW> + i) * 8);
  x.k8 = copy_offset_k8(ks, kBN - 1, lane, w * 16);
  if (kG == 1 || x.nt > 0) issue_tile<kFp8, kW>(0, 0, x.kp, ks, x.vp, vs, 0, x.kend, x.co, x.k8, lane, w, x.g1);
  x.ro = read_offsets(lane);
  if (x.wq_lo >= len) {
    // Every query of this wave lies past the query length (short prompts in
    // a query tile): it does its share of the copies and passes the same
    // barriers as the other waves, and computes nothing.
    for (int t = 0; t <= nloop; ++t) open_interval<kFp8, kW>((t + 1) & 1, (t + 1) % 3, t, x);
    if (kG == 2) {
      __builtin_amdgcn_s_barrier();  // the two barriers of the groups' hand-over
      __builtin_amdgcn_s_barrier();
    }
    return;
  }

  WaveState st;
#pragma unroll
  for (int qb = 0; qb < kNQ; ++qb) {
    const int my_q = x.wq_lo + qb * 32 + col;
    if (kFp8) {
      // 32 code bytes, dims 32*half .. +32, in qreg[qb][0..1]
      const uint8_t *qp = static_cast<const uint8_t *>(q) + (long)b * qs.b + (long)my_q * qs.t +
                          (long)h * qs.h + half * 32;
#pragma unroll
      for (int c = 0; c < 2; ++c)
        st.qreg[qb][c] = my_q < len ? *reinterpret_cast<const bf16x8 *>(qp + c * 16) : bf16x8{};
      st.qreg[qb][2] = st.qreg[qb][3] = bf16x8{};
    } else {
      const uint16_t *qp = static_cast<const uint16_t *>(q) + (long)b * qs.b + (long)my_q * qs.t +
                           (long)h * qs.h + half * 8;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        st.qreg[qb][c] = my_q < len ? *reinterpret_cast<const bf16x8 *>(qp + c * 16) : bf16x8{};
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) st.oacc[db][qb] = f32x16{};
    st.lacc[qb] = f32x4{};
    st.m_run[qb] = -INFINITY;
  }
  st.sel = row_sum_selector(lane);
  // Consume the Q loads here, once: otherwise the loop-header merge leaves
  // them "in flight" for the compiler, which then waits for every outstanding
  // copy (vmcnt(0)) before the first Q use of each unrolled iteration.
#pragma unroll
  for (int qb = 0; qb < kNQ; ++qb)
    asm volatile("" ::"v"(st.qreg[qb][0]), "v"(st.qreg[qb][1]), "v"(st.qreg[qb][2]), "v"(st.qreg[qb][3]));

  // intervals t = 0 .. nt: tile t's K and tile t-1's V; K of tile j is in K
  // slot j % 2, V of tile j in V slot j % 3
  bf16x8 pa[kNQ][4];
  const uint8_t *K0 = g_kring[0], *K1 = g_kring[1], *V0 = g_vring[0], *V1 = g_vring[1], *V2 = g_vring[2];
  if (kG == 2 && x.g1) {
    K0 = g_ring1[0];
    K1 = g_ring1[1];
    V0 = g_ring1[2];
    V1 = g_ring1[3];
    V2 = g_ring1[4];
  }
  for (int t = 0; t <= nloop; t += 6) {
    interval<kCausal, kFp8, kW>(st, pa, K0, V2, 1, 1, t, x);
    if (t + 1 > nloop) break;
    interval<kCausal, kFp8, kW>(st, pa, K1, V0, 0, 2, t + 1, x);
    if (t + 2 > nloop) break;
    interval<kCausal, kFp8, kW>(st, pa, K0, V1, 1, 0, t + 2, x);
    if (t + 3 > nloop) break;
    interval<kCausal, kFp8, kW>(st, pa, K1, V2, 0, 1, t + 3, x);
    if (t + 4 > nloop) break;
    interval<kCausal, kFp8, kW>(st, pa, K0, V0, 1, 2, t + 4, x);
    if (t + 5 > nloop) break;
    interval<kCausal, kFp8, kW>(st, pa, K1, V1, 0, 0, t + 5, x);
  }

#pragma unroll
  for (int qb = 0; qb < kNQ; ++qb) {
    const int my_q = x.wq_lo + qb * 32 + col;
    // row sum of query col: element 0 (col < 16) or 1 (col >= 16) of lane col%16
    const float l0 = __shfl(st.lacc[qb][0], col & 15, 64);
    const float l1 = __shfl(st.lacc[qb][1], col & 15, 64);
    float l_tot = col < 16 ? l0 : l1;
    if constexpr (kG == 2) {
      // The hand-over: once every wave is past its last ring read, the
      // second group's wave w stores its max, row sum and O (column-major by
      // lane, 34 words a lane) in the second rings' memory, and the first
      // group's wave w, which holds the same queries, takes them in.
      static_assert(kNQ == 1 && kW * 34 * 64 * 4 <= 5 * kTileBytes, "hand-over buffer");
      float *xb = reinterpret_cast<float *>(&g_ring1[0][0]) + w * (34 * 64);
      __builtin_amdgcn_s_waitcnt(kVmcnt0Lgkm0);
      __builtin_amdgcn_s_barrier();
      if (x.g1) {
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) xb[(db * 16 + r) * 64 + lane] = st.oacc[db][qb][r];
        xb[32 * 64 + lane] = st.m_run[qb];
        xb[33 * 64 + lane] = l_tot;
      }
      __builtin_amdgcn_s_waitcnt(kVmcnt0Lgkm0);
      __builtin_amdgcn_s_barrier();
      if (x.g1) return;
      const float m0 = st.m_run[qb], m1 = xb[32 * 64 + lane];
      const float mx = fmaxf(m0, m1);
      const float a0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - mx);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mx);
      l_tot = a0 * l_tot + a1 * xb[33 * 64 + lane];
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          st.oacc[db][qb][r] = a0 * st.oacc[db][qb][r] + a1 * xb[(db * 16 + r) * 64 + lane];
    }
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

hipError_t launch_encoder(const void *q, wa_strides qs, const void *k, wa_strides ks,
                          const uint16_t *v, wa_strides vs, uint16_t *o, wa_strides os, int B,
                          int H, int Tq_max, const int32_t *q_lens, int Tk_max,
                          const int32_t *k_lens, int causal, float softmax_scale,
                          const float *q_scale, const float *k_scale, int per_head, hipStream_t stream) {
  const float c_log2 = softmax_scale * kLog2e;
  // one 256-query block per (b, h) for a non-causal range of 129..256
  // queries, so K and V are read once; otherwise 128-query blocks
  const bool wide = !causal && Tq_max > kBMOf<4> && Tq_max <= kBMOf<8>;
  const int bm = wide ? kBMOf<8> : kBMOf<4>;
  const int n_qt = (Tq_max + bm - 1) / bm;
  const long total = (long)B * H * n_qt;
  // Two key groups per block when the grid has no more blocks than the chip
  // has CUs and there are keys enough to share: the same blocks, twice the
  // waves, half the intervals.  (Measured: the single 30-s chunk of 20 heads
  // 25.8 -> 22.0 us, 6 heads 23.7 -> 19.4 us; at 384 and 480 blocks no
  // change, so those keep one group; four groups gained nothing over two.
  // The waves of one block keep their matrix and vector phases together
  // under its barrier, so more waves in a block overlap little of their
  // work.)
  const bool split = !causal && !wide && total <= 256 && Tk_max >= 4 * kBN;
  const dim3 grid((unsigned)((total + 7) / 8 * 8)), block((wide || split ? 8 : 4) * 64);
  const bool fp8 = q_scale != nullptr;
  auto kernel = causal ? (fp8 ? attn_fwd_kernel<true, true, 4, 1> : attn_fwd_kernel<true, false, 4, 1>)
                : wide ? (fp8 ? attn_fwd_kernel<false, true, 8, 1> : attn_fwd_kernel<false, false, 8, 1>)
                : split ? (fp8 ? attn_fwd_kernel<false, true, 4, 2> : attn_fwd_kernel<false, false, 4, 2>)
                        : (fp8 ? attn_fwd_kernel<false, true, 4, 1> : attn_fwd_kernel<false, false, 4, 1>);
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, q, qs, k, ks, v, vs, o, os, H, Tq_max, q_lens,
                     Tk_max, k_lens, c_log2, q_scale, k_scale, per_head, n_qt, (int)total);
  return hipGetLastError();
}

}  // namespace wa
