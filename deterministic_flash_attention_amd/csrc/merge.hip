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
#include "contract.hpp"
#include "kernels.hpp"

namespace detattn {

namespace {

constexpr int kMergeWaves = 4;

template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_kernel(const MergeParams p) {
  static_assert(D % 64 == 0, "one wave covers D in steps of 64 lanes");
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t rh = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  const int64_t nrh = p.rows * p.hq;
  if (rh >= nrh) return;

  float M = -INFINITY, L = 0.0f;
  float A[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) A[k] = 0.0f;
  for (int c = 0; c < p.cmax; ++c) {
    const int64_t slot = (int64_t)c * nrh + rh;
    const float m = p.part_ml[2 * slot];
    const float l = p.part_ml[2 * slot + 1];
    float ca, cb;
    int mode;
    merge_stats(M, L, m, l, ca, cb, mode);
    if (mode != 0) {
      const float* acc = p.part_acc + slot * D;
#pragma unroll
      for (int k = 0; k < PER; ++k) A[k] = merge_elem(A[k], acc[lane + 64 * k], mode, ca, cb);
    }
  }
  uint16_t* o = static_cast<uint16_t*>(p.o) + rh * D;
#pragma unroll
  for (int k = 0; k < PER; ++k) o[lane + 64 * k] = bf16_bits(finalize_elem(A[k], L, p.v_descale));
  if (p.lse != nullptr && lane == 0) p.lse[rh] = finalize_lse(M, L);
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
