// Chunk merge for the split schedule (RL-Kernel page, section 2: "chunks merged
// ascending with the exact FA2 rescale").
//
// One wave per (row, query head) folds that row's chunk partials left to right,
// c = 0, 1, ..., cmax-1, skipping empty partials (m = -inf) without reading
// their accumulators, then finalises and rounds once to bf16.  merge_stats /
// merge_elem / finalize_* are the same functions the monolithic kernels apply
// in registers, so both schedules produce the same bits.  A left fold is
// required: fp32 addition is not associative, so a pairwise tree over chunks
// would differ from the monolithic order.
//
// The loads are taken off the fold's critical path: lane c reads chunk c's
// (m, l) for 64 chunks at once, a ballot names the non-empty ones, and their
// accumulators are read kBatch at a time before the sequential fold over them
// (skipping an empty partial is exactly the fold's own "keep" case).
#include "contract.hpp"
#include "kernels.hpp"

namespace detattn {

namespace {

constexpr int kMergeWaves = 4;

template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_kernel(const MergeParams p) {
  static_assert(D % 64 == 0, "one wave covers D in steps of 64 lanes");
  constexpr int PER = D / 64;
  constexpr int kBatch = 8;  // accumulators in flight per wave
  const int lane = threadIdx.x & 63;
  const int64_t rh = (int64_t)blockIdx.x * kMergeWaves + uniform((int)(threadIdx.x >> 6));
  const int64_t nrh = p.rows * p.hq;
  const bool valid = rh < nrh;  // wave-uniform; the last workgroup may hold idle waves

  float M = -INFINITY, L = 0.0f;
  float A[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) A[k] = 0.0f;
  for (int c0 = 0; valid && c0 < p.cmax; c0 += 64) {
    // Lane c holds the (m, l) of chunk c0 + c; chunks past cmax read as empty.
    float mc = -INFINITY, lc = 0.0f;
    if (c0 + lane < p.cmax) {
      const int64_t slot = (int64_t)(c0 + lane) * nrh + rh;
      mc = p.part_ml[2 * slot];
      lc = p.part_ml[2 * slot + 1];
    }
    uint64_t live = __builtin_amdgcn_ballot_w64(mc != -INFINITY);
    while (live != 0) {
      // The next (up to) kBatch non-empty chunks, ascending: read their
      // accumulators, then fold them one by one.
      int cs[kBatch];
      float acc[kBatch][PER];
      int nb = 0;
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        cs[b] = -1;
        if (live != 0) {
          const int c = (int)__builtin_ctzll(live);
          live &= live - 1;
          cs[b] = c;
          nb = b + 1;
          const float* ap = p.part_acc + ((int64_t)(c0 + c) * nrh + rh) * D;
#pragma unroll
          for (int k = 0; k < PER; ++k) acc[b][k] = ap[lane + 64 * k];
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (b < nb) {
          const float m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                        __builtin_bit_cast(int, mc), cs[b]));
          const float l = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                        __builtin_bit_cast(int, lc), cs[b]));
          float ca, cb;
          bool keep;
          merge_stats(M, L, m, l, ca, cb, keep);
#pragma unroll
          for (int k = 0; k < PER; ++k) A[k] = merge_elem(A[k], acc[b][k], keep, ca, cb);
        }
      }
    }
  }
  // Bounded epilogue: the wave's O row (and lse cell) through descriptors that
  // end at its last valid byte; an idle wave's descriptors hold zero records,
  // and lanes other than lane 0 park their lse store past the bound, so
  // nothing outside the (row, head) cells is ever written.
  const int64_t base = valid ? rh : 0;
  const rsrc_t orr = make_rsrc(static_cast<unsigned char*>(p.o) + base * D * 2,
                               valid ? (uint32_t)(D * 2) : 0u);
  const RowFinal fin(L, p.v_descale);
#pragma unroll
  for (int k = 0; k < PER; ++k) buf_store2(orr, (uint32_t)(lane + 64 * k) * 2u, bf16_bits(fin.elem(A[k])));
  if (p.lse != nullptr) {
    const rsrc_t lr = make_rsrc(p.lse + base, valid ? 4u : 0u);
    buf_store4(lr, lane == 0 ? 0u : kParked, f32_bits(finalize_lse(M, L)));
  }
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int head_dim, hipStream_t stream) {
  const long long nrh = (long long)p.rows * p.hq;
  if (nrh <= 0) return hipSuccess;
  dim3 grid((unsigned)((nrh + kMergeWaves - 1) / kMergeWaves)), block(kMergeWaves * 64);
  switch (head_dim) {
    case 64:
      hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, stream, p);
      break;
    case 128:
      hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, stream, p);
      break;
    case 192:
      hipLaunchKernelGGL(merge_kernel<192>, grid, block, 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace detattn
