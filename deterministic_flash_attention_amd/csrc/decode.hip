// Single-token paged decode over a paged KV cache (page size 16).
//
// Split schedule (RL-Kernel page, section 2: one program per sequence / KV
// head / chunk, then a merge): one workgroup per (sequence, kv-head, 512-key
// chunk) folds its chunk from the empty state for the query heads of the
// kv-head's group and stores the fp32 partial; the merge kernel folds the
// partials in ascending chunk order.  The monolithic schedule folds every chunk
// of a (sequence, kv-head) in registers and stores O; it exists so that tests
// can check that the two schedules agree bit for bit.
//
// The query heads of one group occupy columns 0..G-1 of the 32-column MFMA
// tile; the remaining columns carry zero queries and are never stored.  The
// scores and softmax of a block are computed once, by one wave (the role
// rotates over the D/32 waves block by block, so every SIMD gets its share),
// which publishes P^T and (alpha, m, l) through LDS; every wave then applies
// them to its own 32-wide slice of the output.  The per-block arithmetic is the
// one in contract.hpp on the same operands, which makes a decode row bitwise
// equal to the last row of the prefill of the same sequence.
#include "contract.hpp"
#include "kernels.hpp"

namespace detattn {

namespace {

constexpr int kPageSize = 16;
constexpr int kPagesPerBlock = kBlockKeys / kPageSize;
constexpr int kSplitChunks = 2;  // consecutive chunks per split workgroup

template <int D, bool FP8>
struct DecodeCfg {
  using G = Geom<D, FP8>;
  static constexpr int kWaves = D / 32;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kBlockChunks = kBlockKeys * G::kChunks16;
  static constexpr int kPerThread = kBlockChunks / kThreads;
  static_assert(kPerThread * kThreads == kBlockChunks, "K/V chunks must split evenly");
  // One K and one V stage: a workgroup's next block waits in registers, and
  // the small footprint lets several workgroups share a CU, whose
  // interleaving hides the load latency better than a second stage.  The P
  // slot holds the block's P^T operands (four 1 KB rows of 16 bytes per lane)
  // and one row of (alpha, m, l) per lane.
  static constexpr int kKOff = 0;
  static constexpr int kVOff = G::kKStage;
  static constexpr int kPOff = kVOff + G::kVStage;
  static constexpr int kPRow = kWave * 16;
  static constexpr int kLds = kPOff + 5 * kPRow;
  static_assert(kLds <= 160 * 1024, "LDS budget");
};

template <int D, bool FP8>
struct PagedStager {
  using G = Geom<D, FP8>;
  using C = DecodeCfg<D, FP8>;
  u32x4 kreg[C::kPerThread];
  u32x4 vreg[C::kPerThread];

  // Keys at or past ctx, and keys whose page is outside the cache (base < 0),
  // are staged as zeros, so dead slots (whatever they hold) never reach the
  // MFMA.  page_base(j) returns the element offset of token j's page for this
  // kv head (slot 0), or -1.
  template <typename PageBase>
  __device__ __forceinline__ void load(const unsigned char* kc, const unsigned char* vc, int key0,
                                       int ctx, int64_t token_stride, int tid,
                                       const PageBase& page_base) {
    int64_t off[C::kPerThread];  // byte offset of each chunk in the cache, or -1
#pragma unroll
    for (int u = 0; u < C::kPerThread; ++u) {
      const int x = tid + u * C::kThreads;
      const int r = x / G::kChunks16, col = x % G::kChunks16;
      const int j = key0 + r;
      int64_t byte = -1;
      if (j < ctx) {
        const int64_t base = page_base(j);
        if (base >= 0) byte = (base + (int64_t)(j % kPageSize) * token_stride) * G::kEs + col * 16;
      }
      off[u] = byte;
    }
    // All K loads are issued before the V loads, so the K stage can be
    // written while the V loads are still in flight.
#pragma unroll
    for (int u = 0; u < C::kPerThread; ++u)
      kreg[u] = off[u] >= 0 ? *reinterpret_cast<const u32x4*>(kc + off[u]) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < C::kPerThread; ++u)
      vreg[u] = off[u] >= 0 ? *reinterpret_cast<const u32x4*>(vc + off[u]) : u32x4{0u, 0u, 0u, 0u};
  }
  __device__ __forceinline__ void store_k(unsigned char* ks, int tid) const {
#pragma unroll
    for (int u = 0; u < C::kPerThread; ++u) {
      const int x = tid + u * C::kThreads;
      const int r = x / G::kChunks16, col = x % G::kChunks16;
      lds_store16(ks, (uint32_t)(r * G::kKRow + col * 16), kreg[u]);
    }
  }
  __device__ __forceinline__ void store_v(unsigned char* vs, int tid) const {
#pragma unroll
    for (int u = 0; u < C::kPerThread; ++u) {
      const int x = tid + u * C::kThreads;
      const int r = x / G::kChunks16, col = x % G::kChunks16;
      if constexpr (FP8) {
        const u32x2 a = e4m3x4_to_bf16x4(vreg[u][0]), b = e4m3x4_to_bf16x4(vreg[u][1]);
        const u32x2 c = e4m3x4_to_bf16x4(vreg[u][2]), d = e4m3x4_to_bf16x4(vreg[u][3]);
        const uint32_t o = (uint32_t)(r * G::kVRow + col * 32);
        lds_store16(vs, o, u32x4{a[0], a[1], b[0], b[1]});
        lds_store16(vs, o + 16, u32x4{c[0], c[1], d[0], d[1]});
      } else {
        lds_store16(vs, (uint32_t)(r * G::kVRow + col * 16), vreg[u]);
      }
    }
  }
};

template <int D, bool FP8, bool SPLIT>
__global__ __launch_bounds__(D / 32 * 64) void decode_kernel(const DecodeParams p) {
  using G = Geom<D, FP8>;
  using C = DecodeCfg<D, FP8>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::kLds];
  __shared__ int64_t sPage[kSplitChunks * kBlocksPerChunk * kPagesPerBlock];
  // Q rows live in dynamic LDS sized at launch for the group: (G + 1) rows.
  extern __shared__ __attribute__((aligned(16))) unsigned char sQ[];
  unsigned char* const sK = smem + C::kKOff;
  unsigned char* const sV = smem + C::kVOff;
  unsigned char* const sP = smem + C::kPOff;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  // Work decode: split workgroups own kSplitChunks consecutive chunks of one
  // (sequence, kv head); monolithic workgroups own a whole (sequence, kv head).
  // The kv head varies fastest, so the workgroups reading the same cache pages
  // (one 256-byte row per token and head) run side by side.
  int id = blockIdx.x;
  const int g = id % p.hkv;
  id /= p.hkv;
  int cgrp = 0;
  if constexpr (SPLIT) {
    const int ngroups = (p.cmax + kSplitChunks - 1) / kSplitChunks;
    cgrp = id % ngroups;
    id /= ngroups;
  }
  const int b = id;
  const int grp = p.group;

  int ctx = uniform(p.ctx_lens[b]);
  ctx = max(0, min(ctx, p.max_pages * kPageSize));
  const int nblk = (ctx + kBlockKeys - 1) / kBlockKeys;
  const int nch = (ctx + kChunkKeys - 1) / kChunkKeys;
  // A left window keeps keys [lo, ctx) (the row is the sequence's last token):
  // blocks and chunks wholly below lo are skipped, and their partials are empty.
  const int lo = p.window_left >= 0 ? max(0, ctx - 1 - p.window_left) : 0;
  const int blk_first = lo / kBlockKeys;
  const int chunk_first = blk_first / kBlocksPerChunk;
  int blk_begin = blk_first, blk_end = nblk;
  const int64_t row_head = (int64_t)b * p.hq + (int64_t)g * grp;  // first query head of the group
  const bool ml_writer = (wave == 0) && (h == 0);
  const int64_t chunk_rows = (int64_t)p.batch * p.hq;  // (row, head) slots per chunk

  auto store_ml = [&](int chunk, float mv, float lv) {
    const rsrc_t mlr = make_rsrc(p.part_ml + 2 * ((int64_t)chunk * chunk_rows + row_head),
                                 (uint32_t)grp * 8u);
    buf_store8(mlr, ml_writer ? (uint32_t)n * 8u : kParked, u32x2{f32_bits(mv), f32_bits(lv)});
  };

  if constexpr (SPLIT) {
    const int c0 = cgrp * kSplitChunks;
    const int c1 = min(c0 + kSplitChunks, p.cmax);
    // Chunks past the context, or below the window, hold empty partials
    // (m, l) = (-inf, 0).
    for (int cc = c0; cc < c1; ++cc)
      if (cc >= nch || cc < chunk_first) store_ml(cc, -INFINITY, 0.0f);
    blk_begin = max(c0 * kBlocksPerChunk, blk_first);
    blk_end = min(c1 * kBlocksPerChunk, nblk);
    if (blk_begin >= blk_end) return;
  }

  // The group's G query rows, plus one zero row that the padding columns
  // (n >= G) read, staged in LDS; Q^T operands are read from there per block.
  {
    const rsrc_t qr = make_rsrc(static_cast<const unsigned char*>(p.q) + row_head * G::kRowBytes,
                                (uint32_t)(grp * G::kRowBytes));
    for (int x = tid; x < (grp + 1) * G::kChunks16; x += C::kThreads) {
      const int r = x / G::kChunks16, col = x % G::kChunks16;
      lds_store16(sQ, (uint32_t)(r * G::kQRow + col * 16),
                  buf_load16(qr, (uint32_t)(r * G::kRowBytes + col * 16)));
    }
  }
  const unsigned char* const qrow = sQ + min(n, grp) * G::kQRow;

  const float c = p.c_scale;
  f32x16 acc[1], A[1];
  float m = -INFINITY, l = 0.0f, M = -INFINITY, L = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc[0][i] = 0.0f;
    A[0][i] = 0.0f;
  }

  if (blk_begin < blk_end) {
    const unsigned char* kc = static_cast<const unsigned char*>(p.kc);
    const unsigned char* vc = static_cast<const unsigned char*>(p.vc);
    const int32_t* table = p.page_table + (int64_t)b * p.max_pages;
    const int64_t head_off = (int64_t)g * p.head_stride;
    // Element offset of a page's slot 0 for this kv head, or -1 for a page
    // index outside the cache.
    auto lookup = [&](int page_idx) -> int64_t {
      const int64_t pg = table[page_idx];
      return (pg >= 0 && pg < p.num_pages) ? pg * p.page_stride + head_off : -1;
    };
    const int page0 = blk_begin * kPagesPerBlock;
    if constexpr (SPLIT) {
      // The split workgroup's page-table entries, read once into LDS, so a
      // block's K/V loads wait on one memory round trip instead of two.
      const int npg = min((blk_end - blk_begin) * kPagesPerBlock,
                          (ctx + kPageSize - 1) / kPageSize - page0);
      for (int e = tid; e < npg; e += C::kThreads) sPage[e] = lookup(page0 + e);
      __syncthreads();
    }
    auto page_base = [&](int j) -> int64_t {
      if constexpr (SPLIT) {
        return sPage[j / kPageSize - page0];
      } else {
        return lookup(j / kPageSize);
      }
    };
    // Block pipeline: the K and V of block blk sit in the LDS stages and those
    // of blk+1 in registers.  (1) The block's score wave computes S and the
    // softmax and publishes P^T, alpha, m and l in the P slot; barrier.
    // (2) Every wave takes them, stores K(blk+1) into the K stage (the
    // scores of blk are done) and adds P V to its output slice; barrier.
    // (3) Every wave stores V(blk+1) into the V stage and issues the loads of
    // blk+2.  The barrier of (1) in the next block publishes that V stage.
    PagedStager<D, FP8> stg;
    stg.load(kc, vc, blk_begin * kBlockKeys, ctx, p.token_stride, tid, page_base);
    stg.store_k(sK, tid);
    stg.store_v(sV, tid);
    if (blk_begin + 1 < blk_end)
      stg.load(kc, vc, (blk_begin + 1) * kBlockKeys, ctx, p.token_stride, tid, page_base);
    __syncthreads();
    for (int blk = blk_begin; blk < blk_end;) {
      const int cend = min(blk_end, (blk / kBlocksPerChunk + 1) * kBlocksPerChunk);
      for (; blk < cend; ++blk) {
        const bool more = blk + 1 < blk_end;
        if (wave == blk % C::kWaves) {
          f32x16 s[2];
          qk_scores_qrow<D, FP8>(s, qrow, sK, lane);
          float alpha;
          u32x4 pb[4];
          const int b0 = kBlockKeys * blk;
          if (b0 >= lo && b0 + kBlockKeys <= ctx) {
            softmax_block<kNoMask>(s, h, c, 0, 0, m, l, alpha, pb);
          } else if (b0 >= lo) {
            softmax_block<kMaskHi>(s, h, c, 0, ctx - b0, m, l, alpha, pb);
          } else {
            softmax_block<kMaskLoHi>(s, h, c, lo - b0, ctx - b0, m, l, alpha, pb);
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) lds_store16(sP, (uint32_t)(k * C::kPRow + lane * 16), pb[k]);
          lds_store16(sP, (uint32_t)(4 * C::kPRow + lane * 16),
                      u32x4{f32_bits(alpha), f32_bits(m), f32_bits(l), 0u});
        }
        __syncthreads();  // P^T and the statistics of blk are published
        u32x4 pb[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) pb[k] = lds_load16(sP, (uint32_t)(k * C::kPRow + lane * 16));
        const u32x4 st = lds_load16(sP, (uint32_t)(4 * C::kPRow + lane * 16));
        m = bits_f32(st[1]);
        l = bits_f32(st[2]);
        if (more) stg.store_k(sK, tid);
        pv_accumulate<D, 1, false>(acc, wave, bits_f32(st[0]), pb, sV, lane);
        __syncthreads();  // every wave is done with the P slot and the V stage
        if (more) {
          stg.store_v(sV, tid);
          if (blk + 2 < blk_end)
            stg.load(kc, vc, (blk + 2) * kBlockKeys, ctx, p.token_stride, tid, page_base);
        }
      }
      const int chunk = (blk - 1) / kBlocksPerChunk;  // the chunk just completed
      if constexpr (SPLIT) {
        store_ml(chunk, m, l);
        const rsrc_t ar = make_rsrc(p.part_acc + ((int64_t)chunk * chunk_rows + row_head) * D,
                                    (uint32_t)grp * D * 4u);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * wave + 8 * q4 + 4 * h;
          buf_store16(ar, (uint32_t)(n * D + d) * 4u,
                      u32x4{f32_bits(acc[0][4 * q4 + 0]), f32_bits(acc[0][4 * q4 + 1]),
                            f32_bits(acc[0][4 * q4 + 2]), f32_bits(acc[0][4 * q4 + 3])});
        }
      } else {
        float ca, cb;
        bool keep;
        merge_stats(M, L, m, l, ca, cb, keep);
#pragma unroll
        for (int i = 0; i < 16; ++i) A[0][i] = merge_elem(A[0][i], acc[0][i], keep, ca, cb);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[0][i] = 0.0f;
      m = -INFINITY;
      l = 0.0f;
    }
  }

  if constexpr (!SPLIT) {
    const rsrc_t orr = make_rsrc(static_cast<unsigned char*>(p.o) + row_head * D * 2,
                                 (uint32_t)grp * D * 2u);
    const RowFinal fin(L, p.v_descale);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * wave + 8 * q4 + 4 * h;
      const uint32_t w0 = pack_bf16x2(fin.elem<!FP8>(A[0][4 * q4 + 0]),
                                      fin.elem<!FP8>(A[0][4 * q4 + 1]));
      const uint32_t w1 = pack_bf16x2(fin.elem<!FP8>(A[0][4 * q4 + 2]),
                                      fin.elem<!FP8>(A[0][4 * q4 + 3]));
      buf_store8(orr, (uint32_t)(n * D + d) * 2u, u32x2{w0, w1});
    }
    if (p.lse != nullptr) {
      const rsrc_t lr = make_rsrc(p.lse + row_head, (uint32_t)grp * 4u);
      buf_store4(lr, ml_writer ? (uint32_t)n * 4u : kParked, f32_bits(finalize_lse(M, L)));
    }
  }
}

template <int D, bool FP8>
hipError_t launch_one(const DecodeParams& p, bool split, hipStream_t stream) {
  const long long per = (long long)p.batch * p.hkv *
                        (split ? (p.cmax + kSplitChunks - 1) / kSplitChunks : 1);
  if (per <= 0) return hipSuccess;
  dim3 grid((unsigned)per), block(DecodeCfg<D, FP8>::kThreads);
  const size_t qlds = (size_t)(p.group + 1) * Geom<D, FP8>::kQRow;
  if (split) {
    hipLaunchKernelGGL((decode_kernel<D, FP8, true>), grid, block, qlds, stream, p);
  } else {
    hipLaunchKernelGGL((decode_kernel<D, FP8, false>), grid, block, qlds, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int head_dim, bool fp8, bool split,
                         hipStream_t stream) {
  switch (head_dim) {
    case 64:
      return fp8 ? launch_one<64, true>(p, split, stream) : launch_one<64, false>(p, split, stream);
    case 128:
      return fp8 ? launch_one<128, true>(p, split, stream)
                 : launch_one<128, false>(p, split, stream);
    case 192:
      return fp8 ? launch_one<192, true>(p, split, stream)
                 : launch_one<192, false>(p, split, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace detattn
