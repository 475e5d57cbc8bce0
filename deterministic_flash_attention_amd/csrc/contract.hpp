// The numerical contract shared by every kernel of the library.
//
// The batch-invariant chunked attention forward (RL-Kernel PR "MFMA
// batch-invariant GEMM and chunked Triton attention", section 2) requires that
// prefill, split-KV decode and every batch composition produce bitwise-equal
// rows.  That holds only if every kernel runs the same fp32 operation sequence
// per (query row, key block).  This header is that sequence; the prefill,
// decode and merge kernels call nothing else for arithmetic:
//
//   * keys are consumed in 64-key blocks at absolute positions inside 512-key
//     chunks; each chunk's online softmax starts from the empty state
//     (m = -inf, l = 0, acc = 0);
//   * S^T = K Q^T per block on v_mfma_f32_32x32x16_bf16 with D/16 K-steps, or
//     for e4m3 inputs on v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales) with
//     D/64 K-steps, in ascending order from a zero accumulator; the
//     instruction shape and the K order are part of the contract, as the same
//     page says of its GEMM sibling (section 1);
//   * scores are masked by select (to -inf), never by adding; the block max is
//     m_blk = c * max(raw scores) with c = scale * q_descale * k_descale * log2(e);
//     the row's reference m moves to m_blk only when m_blk > m + 8 (always from
//     the empty state's -inf), so m' is m_blk or m and every p of a chunk is at
//     most about 2^8; alpha = exp2(m - m'), or 1 when m = -inf (the state is empty, l
//     and acc are zeros, and a factor of 0 or 1 leaves them the same bits);
//     p = exp2(fma(s, c, -m')) with v_exp_f32 and one explicit fused
//     multiply-add, a fixed row-sum tree, l = l*alpha + sum(p); a row whose
//     block is fully masked keeps m, l and acc bit for bit (alpha = 1, p = 0,
//     and its empty state uses the safe max 0 so no -inf - -inf appears);
//   * P is rounded to bf16 (nearest even) and acc = (acc*alpha) + P V on
//     v_mfma_f32_32x32x16_bf16, four 16-key K-steps in ascending key order; fp8
//     V is widened exactly to bf16 first.  A wave whose lanes all hold alpha = 1
//     skips the products acc*alpha (x * 1 is x): with the threshold of 8 a
//     chunk's reference rarely moves after its first visible block, so most
//     blocks skip them;
//   * chunk partials (m_c, l_c, acc_c) are folded left to right in ascending
//     chunk order with the exact max/sum rescale (a skipped empty partial, a
//     copy into an empty total, or M' = max(M, m_c), a = exp2(M - M'),
//     b = exp2(m_c - M'), L = L*a + l_c*b, A = A*a + acc_c*b);
//   * O = A / L rounded to nearest (0 for a row with no visible key, L = 0),
//     times v_descale, plus +0 (which turns a -0 into +0 and leaves every other
//     value as it is), rounded once to bf16.  The quotient is formed from the
//     row's correctly rounded reciprocal r = 1 / L (one IEEE division per row)
//     and one remainder correction per element, q0 = A r, e = fma(-q0, L, A),
//     q = fma(e, r, q0): by Markstein's theorem (r within half an ulp of 1/L,
//     q0 within an ulp of A/L, the remainder e exact) q is the correctly
//     rounded A / L whenever the quotient is a normal number.
//
// All code is built with -ffp-contract=off: the compiler fuses no multiply-add.
// The op sequence holds exactly five fused multiply-adds, written explicitly
// and run identically by every kernel: p = exp2(fma(s, c, -m')) in the block
// update, L = fma(L, a, l_c * b) and A = fma(A, a, acc_c * b) in the chunk
// fold, and the two of the finalize correction.  Every other product and sum
// above is a separately rounded fp32 operation.
//
// "Untouched" holds up to the sign of zero: a fully masked block leaves m and
// l bit for bit, and acc too except that an accumulator element that is -0
// (acc * alpha rounds to -0 when alpha underflows) can become +0 by adding the
// block's +0 products.  One tiling computes such a block for a row and another
// skips it, so the finalize step maps -0 to +0; a zero's sign then never
// reaches O, and rows agree bit for bit across tilings and schedules.
#pragma once

#include "common.hpp"

namespace detattn {

constexpr int kBlockKeys = 64;
constexpr int kChunkKeys = 512;
constexpr int kBlocksPerChunk = kChunkKeys / kBlockKeys;
constexpr uint32_t kParked = 0x80000000u;  // store offset past every num_records
// A row's softmax reference moves up only past this margin (log2 units).
constexpr float kRaiseLog2 = 8.0f;

template <int D, bool FP8>
struct Geom {
  static_assert(D % 32 == 0 && D >= 32 && D <= 256, "head_dim must be a multiple of 32");
  static constexpr int kEs = FP8 ? 1 : 2;       // bytes per Q/K/V element in HBM
  static constexpr int kRowBytes = D * kEs;     // one head row of Q/K/V
  // LDS row strides, chosen for gfx950's 64 four-byte banks (256 bytes per
  // cycle).  K rows are read 16 bytes per lane and instruction, 16 lanes per
  // cycle, one row per lane: an odd number of 16-byte units per row puts those
  // rows on distinct banks (and keeps the reads 16-byte aligned).  V rows are read by the transposing
  // read, four rows x 64 bytes per 32-lane cycle: a stride of 64 mod 256 bytes
  // puts the four rows on disjoint banks.
  static constexpr int kQRow = kRowBytes + 16;
  static constexpr int kKRow = kRowBytes + 16;
  static constexpr int kVRow = D * 2 + 64;      // V is staged as bf16
  static constexpr int kKStage = kBlockKeys * kKRow;
  static constexpr int kVStage = kBlockKeys * kVRow;
  static constexpr int kSteps = D / 16;         // QK^T K-steps
  static constexpr int kDTiles = D / 32;        // 32-wide output tiles for PV
  static constexpr int kChunks16 = kRowBytes / 16;  // 16-byte chunks per HBM row
};

// Score element i of key tile t in lane (n, h = lane/32) is the key at offset
// 32t + 16(i/8) + 8h + (i%8) of the block: MFMA row r of tile t holds key
// 32t + sigma(r), sigma swapping bits 2 and 3 of r, so that each lane holds 8
// consecutive keys per 16-key PV step and P feeds the PV MFMA with no lane
// exchange.
__device__ __forceinline__ int key_sigma(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
__device__ __forceinline__ int score_key(int t, int i, int h) {
  return 32 * t + 16 * (i >> 3) + 8 * h + (i & 7);
}
// score_key without the half-wave's 8h: a compile-time constant in 0..63.
constexpr int score_key_base(int t, int i) { return 32 * t + 16 * (i >> 3) + (i & 7); }

// S^T = K_blk Q^T for the 64 keys of the staged block; s[t] holds key tile t.
// qrow points at the lane's query row in LDS (D elements of Q).  K rows sit in
// groups of 16 (one cache page) KPAGE bytes apart, G::kKRow apart inside a
// group; KPAGE = 16 * kKRow is the plain row-major stage.
template <int D, bool FP8, int KPAGE = 16 * Geom<D, FP8>::kKRow>
__device__ __forceinline__ void qk_scores_qrow(f32x16 (&s)[2], const unsigned char* qrow,
                                               const unsigned char* ks, int lane) {
  using G = Geom<D, FP8>;
  static_assert(KPAGE >= 16 * G::kKRow, "a page group holds 16 K rows");
  const int row = key_sigma(lane & 31);
  const int h = lane >> 5;
  const int krow = (row >> 4) * KPAGE + (row & 15) * G::kKRow;  // key tile 0; tile 1 is 2 groups on
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[t][i] = 0.0f;
  if constexpr (FP8) {
    // e4m3: D/64 K-steps of 64 on the 32x32x64 instruction, each lane reading
    // the 32 bytes of its half of the step from its K row and its Q row.
    static_assert(D % 64 == 0, "fp8 head_dim must be a multiple of 64");
#pragma unroll
    for (int st = 0; st < D / 64; ++st) {
      const uint32_t qoff = (uint32_t)(64 * st + 32 * h);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t off = (uint32_t)(krow + 2 * t * KPAGE + 64 * st + 32 * h);
        s[t] = mfma_fp8x64(lds_load16(ks, off), lds_load16(ks, off + 16), lds_load16(qrow, qoff),
                           lds_load16(qrow, qoff + 16), s[t]);
      }
    }
  } else {
#pragma unroll
    for (int st = 0; st < G::kSteps; ++st) {
      const uint32_t qoff = (uint32_t)((16 * st + 8 * h) * G::kEs);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t off = (uint32_t)(krow + 2 * t * KPAGE + (16 * st + 8 * h) * G::kEs);
        s[t] = mfma_bf16(lds_load16(ks, off), lds_load16(qrow, qoff), s[t]);
      }
    }
  }
}

// The lane's Q^T operands for every K-step of qk_scores_qrow, read once from
// its Q row: bf16 one u32x4 per 16-wide step, e4m3 two per 64-wide step.
template <int D, bool FP8>
struct QOperands {
  static constexpr int kCount = FP8 ? 2 * (D / 64) : D / 16;
  u32x4 q[kCount];
  __device__ __forceinline__ void load(const unsigned char* qrow, int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int st = 0; st < kCount; ++st) {
      const uint32_t off = FP8 ? (uint32_t)(64 * (st >> 1) + 32 * h + 16 * (st & 1))
                               : (uint32_t)((16 * st + 8 * h) * 2);
      q[st] = lds_load16(qrow, off);
    }
  }
};

// qk_scores_qrow with the Q^T operands already in registers: the same MFMA
// sequence on the same operand values.
template <int D, bool FP8, int KPAGE = 16 * Geom<D, FP8>::kKRow>
__device__ __forceinline__ void qk_scores_qreg(f32x16 (&s)[2], const QOperands<D, FP8>& qo,
                                               const unsigned char* ks, int lane) {
  using G = Geom<D, FP8>;
  const int row = key_sigma(lane & 31);
  const int h = lane >> 5;
  const int krow = (row >> 4) * KPAGE + (row & 15) * G::kKRow;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[t][i] = 0.0f;
  if constexpr (FP8) {
#pragma unroll
    for (int st = 0; st < D / 64; ++st) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t off = (uint32_t)(krow + 2 * t * KPAGE + 64 * st + 32 * h);
        s[t] = mfma_fp8x64(lds_load16(ks, off), lds_load16(ks, off + 16), qo.q[2 * st],
                           qo.q[2 * st + 1], s[t]);
      }
    }
  } else {
#pragma unroll
    for (int st = 0; st < G::kSteps; ++st) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t off = (uint32_t)(krow + 2 * t * KPAGE + (16 * st + 8 * h) * G::kEs);
        s[t] = mfma_bf16(lds_load16(ks, off), qo.q[st], s[t]);
      }
    }
  }
}

// Same product with the Q^T operands read from the wave's rows of the LDS Q tile
// (qs points at the wave's first row; row stride G::kQRow).
template <int D, bool FP8, int KPAGE = 16 * Geom<D, FP8>::kKRow>
__device__ __forceinline__ void qk_scores_qlds(f32x16 (&s)[2], const unsigned char* qs,
                                               const unsigned char* ks, int lane) {
  qk_scores_qrow<D, FP8, KPAGE>(s, qs + (lane & 31) * Geom<D, FP8>::kQRow, ks, lane);
}

// Combine a value with the one in lane ^ 32.  v_permlane32_swap exchanges the
// upper half-wave of its first operand with the lower half-wave of its second;
// swapping a register with itself leaves the lower half in r[0] and the upper
// half in r[1] of every lane, so both half-waves evaluate lo (op) hi with the
// same operand order and get the same bits.
__device__ __forceinline__ float half_wave_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(f32_bits(x), f32_bits(x), false, false);
  return fmaxf(bits_f32(r[0]), bits_f32(r[1]));
}
__device__ __forceinline__ float half_wave_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(f32_bits(x), f32_bits(x), false, false);
  return bits_f32(r[0]) + bits_f32(r[1]);
}

// Masking of a block: none, keys at block offset >= rel_hi, or keys outside
// [rel_lo, rel_hi) (a sliding window's lower edge).
enum BlockMask { kNoMask = 0, kMaskHi = 1, kMaskLoHi = 2 };

// Online-softmax update of one lane's query column over a 64-key block.
// Returns alpha for the accumulator and P^T as four bf16x8 PV operands.
template <int MASK>
__device__ __forceinline__ void softmax_block(const f32x16 (&s)[2], int h, float c, int rel_lo,
                                              int rel_hi, float& m, float& l, float& alpha,
                                              u32x4 (&pb)[4]) {
  // Phases 0-1: mask by select and row max on the raw dot products.  fl(c*s)
  // is monotonic in s for c > 0, so fl(c * max s) is exactly the max of the
  // scaled scores.  The key bounds are shifted by the half-wave's 8h once, so
  // each test compares score_key - 8h, an inline constant, with them.
  const int hi_h = rel_hi - 8 * h, lo_h = rel_lo - 8 * h;
  float x[2][16];
  float mr0 = -INFINITY, mr1 = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = s[0][i];
    if (MASK == kMaskHi) v = (score_key_base(0, i) < hi_h) ? v : -INFINITY;
    if (MASK == kMaskLoHi) {
      const int key = score_key_base(0, i);
      v = (key >= lo_h && key < hi_h) ? v : -INFINITY;
    }
    x[0][i] = v;
    mr0 = fmaxf(mr0, v);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = s[1][i];
    if (MASK == kMaskHi) v = (score_key_base(1, i) < hi_h) ? v : -INFINITY;
    if (MASK == kMaskLoHi) {
      const int key = score_key_base(1, i);
      v = (key >= lo_h && key < hi_h) ? v : -INFINITY;
    }
    x[1][i] = v;
    mr1 = fmaxf(mr1, v);
  }
  float mr = fmaxf(mr0, mr1);
  // Phase 2: the other half-wave (lane ^ 32) holds the remaining 32 keys.
  mr = half_wave_max(mr);
  const float mb = mr * c;
  // The reference moves only when the block's max passes it by more than
  // kRaiseLog2; otherwise alpha = exp2(0) = 1 and p stays at most about
  // 2^kRaiseLog2.
  const float mn = (mb > m + kRaiseLog2) ? mb : m;
  const bool empty = (mn == -INFINITY);
  const float nms = empty ? 0.0f : -mn;
  alpha = (m == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
  // Phases 3-4: p = exp2(c * s - m'), product and difference in one explicit
  // fused multiply-add (one rounding); masked scores are -inf and give p = 0.
#pragma unroll
  for (int i = 0; i < 16; ++i) x[0][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[0][i], c, nms));
#pragma unroll
  for (int i = 0; i < 16; ++i) x[1][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[1][i], c, nms));
  // Phases 5-6: row-sum tree: pair the two key tiles, halve 16 -> 1, then add
  // the other half-wave's sum.
  float u[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = x[0][i] + x[1][i];
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = u[i] + u[i + 8];
#pragma unroll
  for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) u[i] = u[i] + u[i + w];
  const float rs = half_wave_sum(u[0]);
  l = l * alpha + rs;
  m = mn;
  // Phase 7: P to bf16 (round to nearest even), packed as the PV B operand.
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int t = kk >> 1, b = 8 * (kk & 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) pb[kk][e] = pack_bf16x2(x[t][b + 2 * e], x[t][b + 2 * e + 1]);
  }
}

// acc_j = acc_j * alpha, the first half of the accumulator update.
template <int NT, bool SKIP = true>
__device__ __forceinline__ void rescale_acc(f32x16 (&acc)[NT], float alpha) {
  if (SKIP && __builtin_amdgcn_ballot_w64(alpha != 1.0f) == 0) return;  // x * 1 is x
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = acc[j][i] * alpha;
}

// acc_j += P V for the NT output tiles starting at tile dt0 (acc already rescaled).
// The V^T operand comes from the row-major bf16 V stage through the transposing
// LDS read: lane (group G, i) gets V[16kk + 8h + 0..7][32dt + 16(G%2) + i].
template <int D, int NT>
__device__ __forceinline__ void pv_mfma(f32x16 (&acc)[NT], int dt0, const u32x4 (&pb)[4],
                                        const unsigned char* vs, int lane) {
  constexpr int kVRow = D * 2 + 64;
  const int grp = lane >> 4, li = lane & 15;
  const int h = grp >> 1;
  const int key_r = li >> 2, dq = (li & 3) * 4;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int d = 32 * (dt0 + j) + 16 * (grp & 1) + dq;
      const uint32_t off0 = (uint32_t)((16 * kk + 8 * h + key_r) * kVRow + d * 2);
      const u32x2 lo = __builtin_bit_cast(u32x2, lds_load_tr16(vs, off0));
      const u32x2 hi = __builtin_bit_cast(u32x2, lds_load_tr16(vs, off0 + 4 * kVRow));
      acc[j] = mfma_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[kk], acc[j]);
    }
  }
}

// acc_j = acc_j * alpha + P V: both halves back to back.
template <int D, int NT, bool SKIP = true>
__device__ __forceinline__ void pv_accumulate(f32x16 (&acc)[NT], int dt0, float alpha,
                                              const u32x4 (&pb)[4], const unsigned char* vs,
                                              int lane) {
  rescale_acc<NT, SKIP>(acc, alpha);
  pv_mfma<D, NT>(acc, dt0, pb, vs, lane);
}

// Chunk merge: fold one partial (m, l) into the running (M, L).
// keep: the partial is empty (m = -inf) and the total stays as it is.
// Otherwise each side is scaled by exp2 of its max minus the new max, and an
// empty total gets coefficient 0 instead (its A and L are +0, so the fold then
// copies the partial); the new element is fma(A, ca, acc * cb), two roundings.
__device__ __forceinline__ void merge_stats(float& M, float& L, float m, float l, float& ca,
                                            float& cb, bool& keep) {
  keep = (m == -INFINITY);
  const float Mn = fmaxf(M, m);
  ca = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
  cb = __builtin_amdgcn_exp2f(m - Mn);
  L = keep ? L : __builtin_fmaf(L, ca, l * cb);
  M = Mn;
}
__device__ __forceinline__ float merge_elem(float A, float acc, bool keep, float ca, float cb) {
  return keep ? A : __builtin_fmaf(A, ca, acc * cb);
}

// Finalisation of one row (L >= 1 once any key was visible, else L = 0 and
// A = +0).  UNIT skips the v_descale product, which is exact when v_descale
// is 1 (bf16 inputs), so both forms give the same bits there.
struct RowFinal {
  float L, r, vd;
  __device__ __forceinline__ RowFinal(float L_, float v_descale)
      : L(L_), r(L_ > 0.0f ? 1.0f / L_ : 0.0f), vd(v_descale) {}
  template <bool UNIT = false>
  __device__ __forceinline__ float elem(float A) const {
    const float q0 = A * r;
    const float e = __builtin_fmaf(-q0, L, A);  // exact remainder A - q0 L
    const float q = __builtin_fmaf(e, r, q0);   // RN(A / L); +0 when L = 0
    // x + 0 is x for every x except -0, which becomes +0 (round to nearest even).
    return (UNIT ? q : q * vd) + 0.0f;
  }
};
// Natural-log sum of exp(scale * q.k): M is kept in log2 units.
__device__ __forceinline__ float finalize_lse(float M, float L) {
  return (L > 0.0f) ? (M + __builtin_amdgcn_logf(L)) * 0.693147180559945309f : -INFINITY;
}

}  // namespace detattn
