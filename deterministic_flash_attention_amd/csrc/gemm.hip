// Batch-invariant bf16 GEMM on gfx950 (RL-Kernel PR "MFMA batch-invariant GEMM
// and chunked Triton attention", section 1).
//
// C[M, N] = A[M, K] B[K, N], B = W^T for an [N, K] weight or W itself for a
// [K, N] weight.  The numerical contract, identical for every configuration:
//   - every product runs on v_mfma_f32_32x32x16_bf16 (the pinned MFMA shape);
//     MFMA step s of K block b covers K indices 64 b + 16 s + [0, 16), lane half
//     h supplying K offsets 8 h + [0, 8) for both operands;
//   - K is consumed in ascending 64-wide blocks; the partial of each 1024-wide
//     chunk starts from +0 and chains its blocks' MFMAs in order;
//   - chunk partials are added left to right in fp32 (total = p_0, then
//     total = total + p_c), and the total is rounded once to bf16 (nearest even).
// Every output element depends only on its row of A and its column of B, so the
// tile shape, the wave count, the stage count, the weight layout, M, the row
// stride and the schedule give the same bits.  The split schedule runs one
// workgroup per (tile, chunk), stores fp32 chunk partials and folds them in the
// same left-to-right order in gemm_combine_kernel.
//
// Data movement: each 64-wide K block of the A tile and the B tile is copied
// global -> LDS with direct (buffer_load ... lds) loads, STAGES blocks in flight.
// A and [N, K] B tiles keep 128-byte rows whose 16-byte chunks are XOR-swizzled
// by (row / 2) % 8, so 16 consecutive rows read at one K offset hit 16 distinct
// bank groups; a [K, N] B tile keeps 64 K rows of BN columns, its 16-byte
// granules XOR-swizzled by kn_swizzle(row) so the 4 rows x 64 bytes that half a
// wave's transposing LDS read touches land in 16 distinct bank groups.  Out-of-range rows, columns past a [K, N] row
// end and K past the end read as zero through the buffer range check.
#include "common.hpp"
#include "kernels.hpp"

namespace detattn {

namespace {

constexpr int kGemmBlockK = 64;       // K per block
constexpr int kGemmBlocksPerChunk = 16;  // 1024 / 64
constexpr uint32_t kParkedOff = 0x80000000u;  // past every descriptor (offsets stay below 2^31)

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Granule swizzle of a [K, N] B stage row r holding G = BN / 8 granules of 16
// bytes: row r's base lies (r * G) % 16 granules into a 256-byte bank window,
// and the XOR (which stays inside the row for these G) spreads the four rows a
// half-wave reads over the 16 granules of the window.
template <int G>
__device__ __forceinline__ int kn_swizzle(int r) {
  if constexpr (G % 16 == 0) return 4 * (r & 3);
  else if constexpr (G % 16 == 8) return 4 * ((r >> 1) & 1);
  else return 0;
}

template <int BM, int BN, int WM, int WN, int STAGES, bool KN>
struct GemmCfg {
  static constexpr int kNW = WM * WN;
  static constexpr int kThreads = kNW * 64;
  static constexpr int kTM = BM / WM, kTN = BN / WN;  // wave tile
  static constexpr int kSM = kTM / 32, kSN = kTN / 32;
  static_assert(kTM % 32 == 0 && kTN % 32 == 0, "wave tiles are whole 32x32 MFMA tiles");
  static_assert(STAGES >= 2 && STAGES <= 8, "2 to 8 blocks in flight");
  // A stage: BM rows of 128 bytes; loads per wave rounded up so every wave
  // issues the same count (the surplus lanes write zeros into the stage's tail).
  static constexpr int kAPer = cdiv(BM * 128, 1024 * kNW);
  static constexpr int kAStage = kAPer * kNW * 1024;
  static constexpr int kBRow = KN ? BN * 2 : 128;
  static_assert(!KN || BN % 32 == 0, "a [K, N] row is whole 64-byte column groups");
  static constexpr int kBSlots = kBRow / 16;
  static constexpr int kBRows = KN ? kGemmBlockK : BN;
  static constexpr int kBPer = cdiv(kBRows * kBRow, 1024 * kNW);
  static constexpr int kBStage = kBPer * kNW * 1024;
  static constexpr int kStage = kAStage + kBStage;
  static constexpr int kPer = kAPer + kBPer;  // direct loads per wave per block
  // As many of the requested stages as fit in the 160 KB of LDS and in the
  // 6-bit vmcnt (the loads of kStages - 2 blocks stay in flight at a wait).
  static constexpr int kStagesLds = STAGES * kStage <= 160 * 1024 ? STAGES : 160 * 1024 / kStage;
  static constexpr int kStagesVm = 63 / kPer + 2;
  static constexpr int kStages = kStagesLds < kStagesVm ? kStagesLds : kStagesVm;
  static_assert(kStages >= 2, "two stages must fit");
  static constexpr int kLds = kStages * kStage;
};

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(ahead * PER) for a runtime ahead in [0, MAX].
template <int MAX, int PER>
__device__ __forceinline__ void wait_blocks_ahead(int ahead) {
  if constexpr (MAX <= 0) {
    wait_vm_le<0>();
  } else {
    if (ahead >= MAX) wait_vm_le<MAX * PER>();
    else wait_blocks_ahead<MAX - 1, PER>(ahead);
  }
}

// Workgroup barrier without the implicit memory fence of __syncthreads(): the
// direct loads still in flight are not waited for (wait_vm_le does that for the
// block being published); the asm statements keep LDS accesses on their side.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BM, int BN, int WM, int WN, int STAGES, bool KN, bool SPLIT>
// Two waves per SIMD: four-wave tiles run two workgroups per CU, eight-wave
// tiles one.
__global__ __launch_bounds__(WM * WN * 64, WM * WN >= 8 ? 1 : 2) void gemm_kernel(const GemmParams p) {
  using C = GemmCfg<BM, BN, WM, WN, STAGES, KN>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::kLds];

  // ---- tile of this workgroup -------------------------------------------
  // Consecutive workgroup ids go round-robin to the 8 XCDs; give each XCD a
  // contiguous range of tiles, ordered group_m tile rows at a time (column by
  // column inside a group), so the tiles resident on one XCD share A rows and
  // B columns in its L2.
  const int T = p.tiles_m * p.tiles_n;
  const int bid = blockIdx.x;
  const int q8 = T / 8, r8 = T % 8, x = bid % 8, ix = bid / 8;
  const int t = x < r8 ? x * (q8 + 1) + ix : r8 * (q8 + 1) + (x - r8) * q8 + ix;
  const int per_group = p.group_m * p.tiles_n;
  const int g = t / per_group, tg = t % per_group;
  const int first_m = g * p.group_m;
  const int rows_in_group = min(p.group_m, p.tiles_m - first_m);
  const int tm = first_m + tg % rows_in_group, tn = tg / rows_in_group;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int rows_a = (int)min((int64_t)BM, p.m - m0);
  const int cols_b = (int)min((int64_t)BN, p.n - n0);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave % WM, wn = wave / WM;
  const int l32 = lane & 31, h = lane >> 5;

  // ---- descriptors: one per operand tile, bounded to its valid cells -------
  const int64_t K = p.k;
  const rsrc_t ra = make_rsrc(static_cast<const unsigned char*>(p.a) + m0 * p.lda * 2,
                              (uint32_t)(((int64_t)(rows_a - 1) * p.lda + K) * 2));
  const rsrc_t rb =
      KN ? make_rsrc(static_cast<const unsigned char*>(p.b) + n0 * 2,
                     (uint32_t)(((K - 1) * p.ldb + cols_b) * 2))
         : make_rsrc(static_cast<const unsigned char*>(p.b) + n0 * p.ldb * 2,
                     (uint32_t)(((int64_t)(cols_b - 1) * p.ldb + K) * 2));

  // ---- per-lane direct-load slots -----------------------------------------
  // A (and [N, K] B): LDS position pos = 1024 seg + 16 lane holds row pos / 128,
  // K chunk (pos / 16 % 8) ^ (row / 2 % 8).  kidx is the slot's first K index
  // inside a block (huge for surplus slots, so they always read as zero).
  uint32_t aoff[C::kAPer], boff[C::kBPer];
  int akidx[C::kAPer], bkidx[C::kBPer];
#pragma unroll
  for (int u = 0; u < C::kAPer; ++u) {
    const int pos = 64 * (wave + C::kNW * u) + lane, r = pos >> 3;
    const int c = (pos & 7) ^ ((r >> 1) & 7);
    const bool ok = r < BM;
    aoff[u] = ok ? (uint32_t)(r * p.lda * 2 + 16 * c) : kParkedOff;
    akidx[u] = ok ? 8 * c : (1 << 30);
  }
#pragma unroll
  for (int u = 0; u < C::kBPer; ++u) {
    const int pos = 64 * (wave + C::kNW * u) + lane;
    if constexpr (KN) {
      const int r = pos / C::kBSlots, c = (pos % C::kBSlots) ^ kn_swizzle<C::kBSlots>(r);
      const bool ok = r < kGemmBlockK;
      boff[u] = ok ? (uint32_t)(r * p.ldb * 2 + 16 * c) : kParkedOff;
      bkidx[u] = ok ? r : (1 << 30);
    } else {
      const int r = pos >> 3, c = (pos & 7) ^ ((r >> 1) & 7);
      const bool ok = r < BN;
      boff[u] = ok ? (uint32_t)(r * p.ldb * 2 + 16 * c) : kParkedOff;
      bkidx[u] = ok ? 8 * c : (1 << 30);
    }
  }
  const uint32_t b_kstride = KN ? (uint32_t)(p.ldb * 2) : 2u;  // bytes per K index

  auto issue = [&](int blk, int st) {
    const int k0 = blk * kGemmBlockK;
    unsigned char* sa = smem + st * C::kStage;
    unsigned char* sb = sa + C::kAStage;
#pragma unroll
    for (int u = 0; u < C::kAPer; ++u) {
      const uint32_t off = (int64_t)(k0 + akidx[u]) < K ? aoff[u] + 2u * (uint32_t)k0 : kParkedOff;
      buf_load16_lds(ra, sa + (wave + C::kNW * u) * 1024, off);
    }
#pragma unroll
    for (int u = 0; u < C::kBPer; ++u) {
      const uint32_t off =
          (int64_t)(k0 + bkidx[u]) < K ? boff[u] + b_kstride * (uint32_t)k0 : kParkedOff;
      buf_load16_lds(rb, sb + (wave + C::kNW * u) * 1024, off);
    }
  };

  // ---- LDS read offsets -----------------------------------------------------
  // Row r = (32-aligned base) + l32 at K chunk 2 s + h sits at chunk slot
  // (2 s + h) ^ (l32 / 2 % 8).
  uint32_t coff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) coff[s] = 16u * (uint32_t)((2 * s + h) ^ ((l32 >> 1) & 7));
  const uint32_t a_row = (uint32_t)((wm * C::kTM + l32) * 128);
  const uint32_t b_row = (uint32_t)((wn * C::kTN + l32) * 128);
  // [K, N] B through the transposing read: lane (group grp, li) addresses row
  // 16 s + 8 h + li / 4 (and 4 rows on), column base + 16 (grp % 2) + 4 (li % 4).
  // Those rows agree in their two low bits (li / 4), so one swizzle serves every
  // step; b_col[j] is the swizzled byte column of output tile j.
  const int grp = lane >> 4, li = lane & 15;
  const uint32_t b_tr = (uint32_t)((8 * h + (li >> 2)) * C::kBRow);
  uint32_t b_col[C::kSN];
#pragma unroll
  for (int j = 0; j < C::kSN; ++j) {
    const int cb = (wn * C::kTN + 32 * j + 16 * (grp & 1) + 4 * (li & 3)) * 2;
    b_col[j] = (uint32_t)(16 * ((cb >> 4) ^ kn_swizzle<C::kBSlots>(li >> 2)) + (cb & 15));
  }

  f32x16 acc[C::kSM][C::kSN];
  f32x16 tot[C::kSM][C::kSN];
#pragma unroll
  for (int i = 0; i < C::kSM; ++i)
#pragma unroll
    for (int j = 0; j < C::kSN; ++j) {
      acc[i][j] = f32x16{};
      tot[i][j] = f32x16{};
    }

  // Operands of MFMA step s from stage st: A tiles i, B tiles j of this wave.
  auto read_a = [&](int st, int s, int i) -> u32x4 {
    return lds_load16(smem + st * C::kStage, a_row + 32u * 128u * i + coff[s]);
  };
  auto read_b = [&](int st, int s, int j) -> u32x4 {
    const unsigned char* sb = smem + st * C::kStage + C::kAStage;
    if constexpr (KN) {
      const uint32_t off = b_tr + (uint32_t)(16 * s * C::kBRow) + b_col[j];
      const u32x2 lo = __builtin_bit_cast(u32x2, lds_load_tr16(sb, off));
      const u32x2 hi = __builtin_bit_cast(u32x2, lds_load_tr16(sb, off + 4 * C::kBRow));
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    } else {
      return lds_load16(sb, b_row + 32u * 128u * j + coff[s]);
    }
  };
  // One block, step by step: read a step's operands, run its MFMAs.
  auto compute = [&](int st) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 a[C::kSM], b[C::kSN];
#pragma unroll
      for (int i = 0; i < C::kSM; ++i) a[i] = read_a(st, s, i);
#pragma unroll
      for (int j = 0; j < C::kSN; ++j) b[j] = read_b(st, s, j);
#pragma unroll
      for (int i = 0; i < C::kSM; ++i)
#pragma unroll
        for (int j = 0; j < C::kSN; ++j) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
    }
  };
  // Chunk end: total = p_0, then total = total + p_c; the partial restarts at +0.
  auto fold = [&](int blk, bool last) {
    if (blk % kGemmBlocksPerChunk == kGemmBlocksPerChunk - 1 || last) {
      if constexpr (!SPLIT) {
        const bool first = blk < kGemmBlocksPerChunk;
#pragma unroll
        for (int i = 0; i < C::kSM; ++i)
#pragma unroll
          for (int jj = 0; jj < C::kSN; ++jj) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
              tot[i][jj][e] = first ? acc[i][jj][e] : tot[i][jj][e] + acc[i][jj][e];
            acc[i][jj] = f32x16{};
          }
      }
    }
  };

  // ---- K loop -----------------------------------------------------------------
  const int nchunks = p.nchunks;
  const int c_begin = SPLIT ? (int)blockIdx.y : 0;
  const int c_end = SPLIT ? c_begin + 1 : nchunks;
  const int nblocks_k = (int)((K + kGemmBlockK - 1) / kGemmBlockK);
  const int blk_begin = c_begin * kGemmBlocksPerChunk;
  const int blk_end = min(c_end * kGemmBlocksPerChunk, nblocks_k);
  const int n = blk_end - blk_begin;

  // Block j is published once every wave has its loads of it: at most the loads
  // of the blocks issued after it (ahead of them) may still be in flight.
#pragma unroll
  for (int s = 0; s < C::kStages - 1; ++s)
    if (s < n) issue(blk_begin + s, s);
  for (int j = 0; j < n; ++j) {
    wait_blocks_ahead<C::kStages - 2, C::kPer>(min(C::kStages - 2, n - 1 - j));
    barrier();
    if (j + C::kStages - 1 < n)
      issue(blk_begin + j + C::kStages - 1, (j + C::kStages - 1) % C::kStages);
    compute(j % C::kStages);
    fold(blk_begin + j, j == n - 1);
  }

  // ---- epilogue ---------------------------------------------------------------
  // Descriptors start at the tile's first cell (m0, n0).  Lane (l32, h) of
  // output tile (i, j) holds column 32 j + l32 and rows
  // 32 i + 8 (e / 4) + 4 h + e % 4 of its wave tile in element e.
  if constexpr (SPLIT) {
    const int64_t ld = p.n;
    const rsrc_t rp = make_rsrc(p.part + ((int64_t)c_begin * p.m + m0) * ld + n0,
                                (uint32_t)(((int64_t)(rows_a - 1) * ld + cols_b) * 4));
#pragma unroll
    for (int i = 0; i < C::kSM; ++i)
#pragma unroll
      for (int j = 0; j < C::kSN; ++j) {
        const int col = wn * C::kTN + 32 * j + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = wm * C::kTM + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
          const uint32_t off = col < cols_b ? (uint32_t)((row * ld + col) * 4) : kParkedOff;
          buf_store4(rp, off, f32_bits(acc[i][j][e]));
        }
      }
  } else {
    const int64_t ld = p.ldc;
    const rsrc_t rc = make_rsrc(static_cast<unsigned char*>(p.c) + (m0 * ld + n0) * 2,
                                (uint32_t)(((int64_t)(rows_a - 1) * ld + cols_b) * 2));
#pragma unroll
    for (int i = 0; i < C::kSM; ++i)
#pragma unroll
      for (int j = 0; j < C::kSN; ++j) {
        const int col = wn * C::kTN + 32 * j + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = wm * C::kTM + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
          const uint32_t off = col < cols_b ? (uint32_t)((row * ld + col) * 2) : kParkedOff;
          buf_store2(rc, off, bf16_bits(tot[i][j][e]));
        }
      }
  }
}

// Split schedule, second pass: C = bf16(((p_0 + p_1) + p_2) + ...), the same
// left fold the monolithic kernel runs in registers.  A workgroup owns 1024
// consecutive columns of one row (one thread per 4 columns), so its
// descriptors are uniform: the partial rows are read and the C row stored
// through descriptors whose num_records ends at column n, and threads past the
// row's last column quad park their offsets beyond it.
constexpr int kCombineThreads = 256;
constexpr int kCombineCols = 4 * kCombineThreads;

__global__ __launch_bounds__(kCombineThreads) void gemm_combine_kernel(const GemmParams p) {
  const int64_t col_blocks = (p.n + kCombineCols - 1) / kCombineCols;
  const int64_t row = (int64_t)blockIdx.x / col_blocks;
  const int64_t col = (int64_t)(blockIdx.x % col_blocks) * kCombineCols + 4 * threadIdx.x;
  const int64_t plane = p.m * p.n;
  const uint32_t in_off = col < p.n ? (uint32_t)(col * 4) : kParkedOff;
  f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c = 0; c < p.nchunks; ++c) {
    const rsrc_t rp = make_rsrc(p.part + c * plane + row * p.n, (uint32_t)(p.n * 4));
    const f32x4 v = __builtin_bit_cast(f32x4, buf_load16(rp, in_off));
    if (c == 0) {
      t = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = t[e] + v[e];
    }
  }
  u32x2 o;
  o[0] = pack_bf16x2(t[0], t[1]);
  o[1] = pack_bf16x2(t[2], t[3]);
  const rsrc_t rc = make_rsrc(static_cast<unsigned char*>(p.c) + row * p.ldc * 2, (uint32_t)(p.n * 2));
  buf_store8(rc, col < p.n ? (uint32_t)(col * 2) : kParkedOff, o);
}

template <int BM, int BN, int WM, int WN, int STAGES>
hipError_t launch_cfg(const GemmParams& p0, bool kn, bool split, hipStream_t stream) {
  GemmParams p = p0;
  p.tiles_m = (int32_t)((p.m + BM - 1) / BM);
  p.tiles_n = (int32_t)((p.n + BN - 1) / BN);
  p.group_m = max(1, min(p.group_m, p.tiles_m));
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n), split ? (unsigned)p.nchunks : 1u);
  const dim3 block(WM * WN * 64);
  if (kn) {
    if (split) hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, STAGES, true, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, STAGES, true, false>), grid, block, 0, stream, p);
  } else {
    if (split) hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, STAGES, false, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, STAGES, false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

// Tile configurations.  The two large ones run two workgroups of four waves on
// each CU (80 KB and 64 KB of LDS), so one workgroup's barrier and load waits
// overlap the other's MFMAs; the small ones serve few rows (decode), where a
// workgroup streams one chunk of the weight and more blocks in flight hide the
// memory latency.
int gemm_num_configs() { return 6; }

void gemm_config_tile(int config, int* bm, int* bn) {
  static const int kTiles[6][2] = {{128, 192}, {128, 128}, {64, 64}, {32, 64}, {32, 32}, {256, 192}};
  *bm = kTiles[config][0];
  *bn = kTiles[config][1];
}

hipError_t launch_gemm(const GemmParams& p, int config, bool kn, bool split, hipStream_t stream) {
  if (p.m > 0 && p.n > 0 && p.nchunks > 0) {
    hipError_t e = hipSuccess;
    switch (config) {
      case 0: e = launch_cfg<128, 192, 2, 2, 2>(p, kn, split, stream); break;
      case 1: e = launch_cfg<128, 128, 2, 2, 2>(p, kn, split, stream); break;
      case 2: e = launch_cfg<64, 64, 2, 2, 6>(p, kn, split, stream); break;
      case 3: e = launch_cfg<32, 64, 1, 2, 8>(p, kn, split, stream); break;
      case 4: e = launch_cfg<32, 32, 1, 1, 8>(p, kn, split, stream); break;
      case 5: e = launch_cfg<256, 192, 4, 2, 2>(p, kn, split, stream); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || !split) return e;
  }
  // Split combine; also the whole job when K = 0 (C = +0).
  if (p.m > 0 && p.n > 0 && (split || p.nchunks == 0)) {
    const int64_t blocks = p.m * ((p.n + kCombineCols - 1) / kCombineCols);
    hipLaunchKernelGGL(gemm_combine_kernel, dim3((unsigned)blocks), dim3(kCombineThreads), 0,
                       stream, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace detattn
