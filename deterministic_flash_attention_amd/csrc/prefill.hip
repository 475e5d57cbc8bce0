// Prefill / full-sequence forward over packed variable-length sequences.
//
// One workgroup owns a tile of 32*NW query rows of one (sequence, query head).
// The Q tile is staged once in its own LDS region, from which each wave reads
// its 32 rows' Q^T operands; K and V blocks of 64 keys stream through two LDS
// stages that are disjoint from the Q region (the ffpa-attn fp8 D=192 page
// shows what a K stage landing in a live Q tile does).  Keys are folded in
// 512-key chunks exactly as contract.hpp prescribes.
//
// bf16 K and V (and e4m3 K from packed rows) go from HBM straight into the
// padded LDS stages (buffer loads with an LDS destination, no staging
// registers); e4m3 V goes through registers because it is widened to bf16 on
// the way.  Block schedules:
//   ping-pong   eight bf16 waves, D <= 128: the two halves of the workgroup
//               alternate (one in its MFMA phase while the other runs its
//               softmax, two barriers per block);
//   pair        e4m3 D = 192 from packed rows: of the two waves sharing a SIMD
//               and 32 query rows, one computes the scores and softmax once
//               for both and hands P over through LDS;
//   lockstep    the other layouts: every wave runs the block with block j+1
//               in flight and one barrier per block.
// Over a paged cache a single-token sequence packs the query heads of its kv
// group into one tile set; with a workspace its chunks spread over otherwise
// idle workgroups, whose bf16 tiles run a block loop of their own (three K/V
// stages, the staging on the second half of the waves).
//
// Schedules (RL-Kernel page, section 2):
//   monolithic  the workgroup folds every chunk of its tile in registers and
//               stores bf16 O (and lse);
//   split       one workgroup per (tile, head, chunk) stores the fp32 chunk
//               partial; the merge kernel folds the partials.  Both run the
//               same per-chunk code, so the merged result is bit-identical.
//
// Stores are bounded by buffer descriptors whose num_records ends at the last
// valid row of the sequence (FlyDSL conv3d and aiter MQA-logits pages): padded
// tail rows of a tile are dropped by the hardware range check, so they can
// never land on the next sequence's rows.
#include <type_traits>

#include "contract.hpp"

#include "kernels.hpp"

namespace detattn {

namespace {

template <int D, bool FP8, int NW, bool PAGED = false>
struct PrefillCfg {
  using G = Geom<D, FP8>;
  // K/V staged by direct global -> LDS loads for bf16 (paged: up to D = 128,
  // where the page-aligned stages fit); otherwise through registers (fp8 V is
  // widened on the way).
  static constexpr bool kDirect = !FP8 && (!PAGED || D <= 128);
  // e4m3 from packed rows: K by direct loads (no widening), V through
  // registers (widened to bf16 on the way).
  static constexpr bool kDirectK = FP8 && !PAGED;
  static constexpr int kThreads = NW * kWave;
  // Wide heads on eight waves split D: waves w and w + kQGroups own the same 32
  // query rows (both compute its scores and softmax) and each keeps half of
  // the output columns, so a wave's accumulator and running total fit the 256
  // registers of two waves per SIMD.
  static constexpr int kDSplit = (D > 128 && NW == 8) ? 2 : 1;
  static constexpr int kQGroups = NW / kDSplit;
  static constexpr int kTileRows = 32 * kQGroups;
  static constexpr int kQBytes = kTileRows * G::kQRow;
  static constexpr int kBlockChunks = kBlockKeys * G::kChunks16;  // 16-B chunks per K block
  static constexpr int kPerThread = (kBlockChunks + kThreads - 1) / kThreads;
  // K rows in groups of 16 (one cache page); a directly staged paged K stage
  // pads each group to whole 1 KB segments so that no segment spans two pages.
  static constexpr int kKPage =
      (PAGED && kDirect) ? (16 * G::kKRow + 1023) / 1024 * 1024 : 16 * G::kKRow;
  static constexpr int kKStage = 4 * kKPage;
  static constexpr int kVStage = G::kVStage;  // 16 V rows are whole 1 KB segments
  // e4m3 wide heads from packed rows run the score/PV pair schedule: of the two
  // waves that share a SIMD and a 32-row query group, the score wave (w < 4)
  // computes the scores and the softmax of each block once and hands P and
  // (alpha, m, l) to its PV wave (w + 4) through LDS, in two alternating P slots.
  static constexpr bool kPairPC = FP8 && !PAGED && kDSplit == 2;
  static constexpr int kPairTilesS = 2;                   // output tiles of a score wave
  static constexpr int kPairTilesV = D / 32 - kPairTilesS;  // and of its PV wave
  static constexpr int kPRow = kWave * 16;                // one u32x4 per lane
  static constexpr int kPSlot = 4 * kPRow + 32 * 16;      // P^T + (alpha, m, l) per query column
  static constexpr int kKOff = kQBytes;
  static constexpr int kVOff = kKOff + 2 * kKStage;
  static constexpr int kEnd = kVOff + 2 * kVStage;
  // Pair schedule layout: three K stages (K reaches LDS two blocks ahead), two
  // V stages and the P slots; no Q tile (the score waves read their Q^T operands
  // straight into registers).
  static constexpr int kPcKStages = 3;
  static constexpr int kPcKOff = 0;
  static constexpr int kPcVOff = kPcKOff + kPcKStages * kKStage;
  static constexpr int kPcPOff = kPcVOff + 2 * kVStage;
  static constexpr int kPcEnd = kPcPOff + 2 * kQGroups * kPSlot;
  static constexpr int kLds = kPairPC ? kPcEnd : kEnd;
  // Q tile, the K stages, the V stages and the P slots are disjoint byte ranges.
  static_assert(kKOff >= kQBytes && kVOff >= kKOff + 2 * kKStage && kEnd >= kVOff + 2 * kVStage,
                "LDS regions overlap");
  static_assert(kPcVOff >= kPcKOff + kPcKStages * kKStage && kPcPOff >= kPcVOff + 2 * kVStage,
                "LDS regions overlap");
  static_assert(kDirect || kKPage == 16 * G::kKRow, "register staging writes row-major stages");
};

__device__ __forceinline__ uint32_t extent_bytes(int64_t nrows, int64_t row_bytes,
                                                 int64_t width_bytes, int64_t avail) {
  if (nrows <= 0 || avail <= 0) return 0u;
  int64_t e = (nrows - 1) * row_bytes + width_bytes;
  if (e > avail) e = avail;
  if (e > 0x7FFFFFFF) e = 0x7FFFFFFF;
  return (uint32_t)e;
}

// Global -> registers -> LDS staging of a 64-key K block and a 64-key V block
// (not necessarily the same block; either may be absent, uniformly per call).
template <int D, bool FP8, int NW>
struct KVStager {
  using G = Geom<D, FP8>;
  using C = PrefillCfg<D, FP8, NW>;
  u32x4 kreg[C::kPerThread];
  u32x4 vreg[C::kPerThread];

  __device__ __forceinline__ void load(rsrc_t kr, int kkey0, bool kon, rsrc_t vr, int vkey0,
                                       bool von, uint32_t row_bytes, int tid) {
#pragma unroll
    for (int u = 0; u < C::kPerThread; ++u) {
      const int x = tid + u * C::kThreads;
      if (C::kPerThread * C::kThreads == C::kBlockChunks || x < C::kBlockChunks) {
        const int r = x / G::kChunks16, col = x % G::kChunks16;
        // kkey0 / vkey0 are relative to the descriptors' base row and may be
        // negative; the offset then wraps past every descriptor (zeros).
        if (kon) kreg[u] = buf_load16(kr, (uint32_t)((int64_t)(kkey0 + r) * row_bytes) + (uint32_t)col * 16u);
        if (von) vreg[u] = buf_load16(vr, (uint32_t)((int64_t)(vkey0 + r) * row_bytes) + (uint32_t)col * 16u);
      }
    }
  }
  // Paged caches: key j sits at element offset page_base(j) + (j % 16) *
  // token_stride, page_base(j) being its page's slot-0 offset for this kv head,
  // or -1 for a page index outside the cache.  Keys at or past lk and keys on
  // such pages are staged as zeros, so dead cache slots never reach the MFMA.
  template <typename PageBase>
  __device__ __forceinline__ void load_paged(const unsigned char* kc, const unsigned char* vc,
                                             int key0, int lk, int64_t token_stride,
                                             const PageBase& page_base, int tid) {
#pragma unroll
    for (int u = 0; u < C::kPerThread; ++u) {
      const int x = tid + u * C::kThreads;
      if (C::kPerThread * C::kThreads == C::kBlockChunks || x < C::kBlockChunks) {
        const int r = x / G::kChunks16, col = x % G::kChunks16;
        const int j = key0 + r;
        u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
        if (j < lk) {
          const int64_t base = page_base(j);
          if (base >= 0) {
            const int64_t byte = (base + (int64_t)(j % 16) * token_stride) * G::kEs + col * 16;
            kv = *reinterpret_cast<const u32x4*>(kc + byte);
            vv = *reinterpret_cast<const u32x4*>(vc + byte);
          }
        }
        kreg[u] = kv;
        vreg[u] = vv;
      }
    }
  }
  __device__ __forceinline__ void store(unsigned char* ks, bool kon, unsigned char* vs, bool von,
                                        int tid) const {
#pragma unroll
    for (int u = 0; u < C::kPerThread; ++u) {
      const int x = tid + u * C::kThreads;
      if (C::kPerThread * C::kThreads == C::kBlockChunks || x < C::kBlockChunks) {
        const int r = x / G::kChunks16, col = x % G::kChunks16;
        if (kon) lds_store16(ks, (uint32_t)(r * G::kKRow + col * 16), kreg[u]);
        if (!von) continue;
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
  }
};

// Direct staging of bf16 K and V blocks of a packed sequence into their padded
// stages.  A stage is a whole number of 1 KB segments; one wave instruction
// fills one segment, lane i the 16-byte slot i of it.  A slot is a 16-byte
// chunk of a K/V row or a row's padding; padding lanes load from a parked
// offset, which the range check turns into zeros.  Rows past the sequence
// read as zeros (the descriptors end at its last key row).
template <int D, int NW, bool FP8 = false>
struct DirectStager {
  using G = Geom<D, FP8>;
  static constexpr int kKSlots = G::kKRow / 16;  // slots per padded row = segments per stage
  static constexpr int kVSlots = G::kVRow / 16;  // (issue_v: bf16 only)
  static constexpr int kKPer = (kKSlots + NW - 1) / NW;  // segments per wave
  static constexpr int kVPer = (kVSlots + NW - 1) / NW;
  static_assert(G::kKRow % 16 == 0 && G::kVRow % 16 == 0, "padded rows must be whole slots");
  static_assert(kBlockKeys == 64 && kKSlots * 1024 == G::kKStage && kVSlots * 1024 == G::kVStage,
                "a stage must be whole 1 KB segments");
  uint32_t koff[kKPer];  // this lane's byte offset inside a block, per segment of this wave
  uint32_t voff[kVPer];
  rsrc_t kr, vr;
  uint32_t row_bytes;
  int kbase;  // key row at which the descriptors start

  static __device__ __forceinline__ uint32_t slot_offset(int seg, int lane, int slots,
                                                         uint32_t row_bytes) {
    const int s = 64 * seg + lane, row = s / slots, c = s % slots;
    return c < G::kChunks16 ? (uint32_t)row * row_bytes + 16u * (uint32_t)c : kParked;
  }
  __device__ __forceinline__ void init(int wave, int lane, rsrc_t k, rsrc_t v, uint32_t rb,
                                       int base) {
    kr = k;
    vr = v;
    row_bytes = rb;
    kbase = base;
#pragma unroll
    for (int u = 0; u < kKPer; ++u) koff[u] = slot_offset(wave + u * NW, lane, kKSlots, rb);
#pragma unroll
    for (int u = 0; u < kVPer; ++u) voff[u] = slot_offset(wave + u * NW, lane, kVSlots, rb);
  }
  __device__ __forceinline__ void prefetch(int, int) {}  // nothing to look up
  __device__ __forceinline__ void latch() {}
  // Byte offset of block blk's first row from the descriptors' base row kbase.
  // It is negative (wrapping to a huge unsigned value) for the block holding
  // kbase when kbase is not block-aligned: rows below kbase then fail the range
  // check and read zeros, which is the window's lower bound done in hardware.
  // Pad lanes add it to the constant parked offset, never to a multiple of the
  // window: 0x80000000 - 63 rows stays past every descriptor, because key rows
  // (plus a block) fit 31 bits.
  __device__ __forceinline__ uint32_t block_offset(int blk) const {
    return (uint32_t)((int64_t)(blk * kBlockKeys - kbase) * row_bytes);
  }
  __device__ __forceinline__ void issue_k(int blk, unsigned char* ks, int wave) const {
    const uint32_t blk_off = block_offset(blk);
#pragma unroll
    for (int u = 0; u < kKPer; ++u) {
      const int seg = wave + u * NW;
      if (kKPer * NW == kKSlots || seg < kKSlots) buf_load16_lds(kr, ks + seg * 1024, koff[u] + blk_off);
    }
  }
  __device__ __forceinline__ void issue_v(int blk, unsigned char* vs, int wave) const {
    const uint32_t blk_off = block_offset(blk);
#pragma unroll
    for (int u = 0; u < kVPer; ++u) {
      const int seg = wave + u * NW;
      if (kVPer * NW == kVSlots || seg < kVSlots) buf_load16_lds(vr, vs + seg * 1024, voff[u] + blk_off);
    }
  }
};

// Direct staging of bf16 K and V blocks from a paged cache.  A block is four
// 16-token pages; each stage holds them as four page regions of whole 1 KB
// segments (K rows padded to KPAGE per region, V regions exactly 16 rows), so
// every segment comes from one page.  NW/4 waves share a page region, so each
// wave reads one page per operand and block, through a descriptor based at
// the page's slot 0 for this kv head whose num_records ends at the page's last
// live token.  Slots past it, padding slots and pages whose table entry lies
// outside the cache (a descriptor of zero records) read as zeros.
template <int D, int NW, int KPAGE>
struct PagedDirectStager {
  using G = Geom<D, false>;
  static constexpr int kWavesPerPage = NW / 4;
  static constexpr int kKSegs = KPAGE / 1024;          // segments per page region
  static constexpr int kVSegs = 16 * G::kVRow / 1024;
  static constexpr int kKSlots = G::kKRow / 16;        // slots per padded row
  static constexpr int kVSlots = G::kVRow / 16;
  static constexpr int kKPer = (kKSegs + kWavesPerPage - 1) / kWavesPerPage;  // per wave
  static constexpr int kVPer = (kVSegs + kWavesPerPage - 1) / kWavesPerPage;
  static_assert(NW % 4 == 0, "waves are dealt evenly to the four pages of a block");
  static_assert(KPAGE % 1024 == 0 && (16 * G::kVRow) % 1024 == 0 && KPAGE >= 16 * G::kKRow,
                "page regions must be whole 1 KB segments holding 16 rows");
  uint32_t koff[kKPer];  // this lane's byte offset inside the page, per segment of this wave
  uint32_t voff[kVPer];
  const unsigned char* kc;  // caches at this kv head's offset
  const unsigned char* vc;
  const int32_t* table;     // this sequence's page-table row
  int64_t num_pages;
  int64_t page_bytes;
  uint32_t token_bytes;
  int lk;
  int max_pages;
  int page;                 // this wave's page of every block (0..3)
  int sub;                  // and its rank among the waves of that page
  int32_t kent, vent;       // table entries of this wave's pages of the next K and V blocks,
                            // as loaded
  int32_t kpg, vpg;         // the same, scalar, for the issue that uses them

  static __device__ __forceinline__ uint32_t slot_offset(int sp, int lane, int slots,
                                                         uint32_t token_bytes) {
    const int s = 64 * sp + lane, row = s / slots, c = s % slots;
    return (row < 16 && c < G::kChunks16) ? (uint32_t)row * token_bytes + 16u * (uint32_t)c
                                          : kParked;
  }
  __device__ __forceinline__ void init(int wave, int lane, const unsigned char* k,
                                       const unsigned char* v, const int32_t* tab, int64_t npages,
                                       int64_t pbytes, uint32_t tbytes, int keys, int mpages) {
    kc = k;
    vc = v;
    table = tab;
    num_pages = npages;
    page_bytes = pbytes;
    token_bytes = tbytes;
    lk = keys;
    max_pages = mpages;
    page = wave / kWavesPerPage;
    sub = wave % kWavesPerPage;
#pragma unroll
    for (int u = 0; u < kKPer; ++u) koff[u] = slot_offset(sub + u * kWavesPerPage, lane, kKSlots, tbytes);
#pragma unroll
    for (int u = 0; u < kVPer; ++u) voff[u] = slot_offset(sub + u * kWavesPerPage, lane, kVSlots, tbytes);
  }
  // Read this wave's table entries of K block kblk and V block vblk, to be
  // issued next; indices are clamped into the table row (entries of pages
  // without a live token are never used).
  // The entries stay in vector registers until latch(), at the start of the
  // staging event that uses them, before that event issues any load:
  // converting them right after the loads would wait for every load issued
  // before them, the block's K/V loads included.
  __device__ __forceinline__ void prefetch(int kblk, int vblk) {
    kent = table[max(0, min(kblk * 4 + page, max_pages - 1))];
    vent = table[max(0, min(vblk * 4 + page, max_pages - 1))];
  }
  // One entry per wave (its page): scalar, so the page descriptors are too.
  __device__ __forceinline__ void latch() {
    kpg = uniform(kent);
    vpg = uniform(vent);
  }
  // Descriptor of this wave's page of block blk, whose table entry is pg.
  __device__ __forceinline__ rsrc_t page_rsrc(const unsigned char* cache, int blk,
                                              int32_t pg) const {
    const int live = min(16, lk - (blk * kBlockKeys + 16 * page));
    const bool ok = live > 0 && pg >= 0 && (int64_t)pg < num_pages;
    return make_rsrc(cache + (ok ? (int64_t)pg * page_bytes : 0),
                     ok ? (uint32_t)(live - 1) * token_bytes + (uint32_t)G::kRowBytes : 0u);
  }
  // The same descriptor as words, for buf_load16_lds_async.
  __device__ __forceinline__ u32x4 page_words(const unsigned char* cache, int blk,
                                              int32_t pg) const {
    const int live = min(16, lk - (blk * kBlockKeys + 16 * page));
    const bool ok = live > 0 && pg >= 0 && (int64_t)pg < num_pages;
    return rsrc_words(cache + (ok ? (int64_t)pg * page_bytes : 0),
                      ok ? (uint32_t)(live - 1) * token_bytes + (uint32_t)G::kRowBytes : 0u);
  }
  // Table entries of this wave's page of blocks [blk0, blk0 + 64), lane i
  // holding block blk0 + i's (clamped into the table row like prefetch).
  __device__ __forceinline__ int32_t entries(int blk0, int lane) const {
    return table[max(0, min((blk0 + lane) * 4 + page, max_pages - 1))];
  }
  // A scalar table entry for the next issue_k / issue_v.
  __device__ __forceinline__ void use_entry(int32_t pg) { kpg = vpg = pg; }
  // Loads one issue_k + issue_v makes for a wave of rank sb in its page.
  static constexpr int loads_per_block(int sb) {
    int n = 0;
    for (int u = 0; u < kKPer; ++u) n += (kKPer * kWavesPerPage == kKSegs || sb + u * kWavesPerPage < kKSegs);
    for (int u = 0; u < kVPer; ++u) n += (kVPer * kWavesPerPage == kVSegs || sb + u * kWavesPerPage < kVSegs);
    return n;
  }
  // Issue K block blk / V block blk: the last prefetch (or use_entry) must
  // have named it.  ASYNC issues the loads from inline assembly (they stay in
  // flight past later LDS reads; the caller waits for them).
  template <bool ASYNC = false>
  __device__ __forceinline__ void issue_k(int blk, unsigned char* ks, int) const {
    unsigned char* const base = ks + page * KPAGE;
    if constexpr (ASYNC) {
      const u32x4 rw = page_words(kc, blk, kpg);
#pragma unroll
      for (int u = 0; u < kKPer; ++u) {
        const int sp = sub + u * kWavesPerPage;
        if (kKPer * kWavesPerPage == kKSegs || sp < kKSegs) buf_load16_lds_async(rw, base + sp * 1024, koff[u]);
      }
    } else {
      const rsrc_t r = page_rsrc(kc, blk, kpg);
#pragma unroll
      for (int u = 0; u < kKPer; ++u) {
        const int sp = sub + u * kWavesPerPage;
        if (kKPer * kWavesPerPage == kKSegs || sp < kKSegs) buf_load16_lds(r, base + sp * 1024, koff[u]);
      }
    }
  }
  template <bool ASYNC = false>
  __device__ __forceinline__ void issue_v(int blk, unsigned char* vs, int) const {
    unsigned char* const base = vs + page * (16 * G::kVRow);
    if constexpr (ASYNC) {
      const u32x4 rw = page_words(vc, blk, vpg);
#pragma unroll
      for (int u = 0; u < kVPer; ++u) {
        const int sp = sub + u * kWavesPerPage;
        if (kVPer * kWavesPerPage == kVSegs || sp < kVSegs) buf_load16_lds_async(rw, base + sp * 1024, voff[u]);
      }
    } else {
      const rsrc_t r = page_rsrc(vc, blk, vpg);
#pragma unroll
      for (int u = 0; u < kVPer; ++u) {
        const int sp = sub + u * kWavesPerPage;
        if (kVPer * kWavesPerPage == kVSegs || sp < kVSegs) buf_load16_lds(r, base + sp * 1024, voff[u]);
      }
    }
  }
};

// Split schedule epilogue: the chunk partial of this wave's query row and
// output tiles [dt0, dt0 + NT): (m, l) by one lane per row (lane half 0 of the
// wave holding tile 0), acc by every lane; both through descriptors that end at
// the sequence's last row.
template <int D, int NT>
__device__ __forceinline__ void store_partial(const PrefillParams& p, const f32x16 (&acc)[NT],
                                              float m, float l, int dt0, int chunk,
                                              int64_t q_start, int head, int nrows, int64_t rs,
                                              int qrow, int h) {
  const int64_t ml_head = ((int64_t)chunk * p.total_q + q_start) * p.hq + head;
  const rsrc_t mlr = make_rsrc(p.part_ml + 2 * ml_head,
                               extent_bytes(nrows, rs * 8, 8,
                                            ((int64_t)(chunk + 1) * p.total_q * p.hq - ml_head) * 8));
  buf_store8(mlr, (h || dt0) ? kParked : (uint32_t)qrow * (uint32_t)(rs * 8),
             u32x2{f32_bits(m), f32_bits(l)});
  const int64_t acc_head = ml_head * D;
  const rsrc_t ar = make_rsrc(p.part_acc + acc_head,
                              extent_bytes(nrows, rs * D * 4, D * 4,
                                           ((int64_t)(chunk + 1) * p.total_q * p.hq * D - acc_head) * 4));
  const uint32_t rowoff = (uint32_t)qrow * (uint32_t)(rs * D * 4);
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * (dt0 + j) + 8 * q4 + 4 * h;
      buf_store16(ar, rowoff + (uint32_t)d * 4u,
                  u32x4{f32_bits(acc[j][4 * q4 + 0]), f32_bits(acc[j][4 * q4 + 1]),
                        f32_bits(acc[j][4 * q4 + 2]), f32_bits(acc[j][4 * q4 + 3])});
    }
}

// Monolithic epilogue: O = A / L (times v_descale) for output tiles
// [dt0, dt0 + NT) rounded once to bf16, and lse from the wave holding tile 0.
// UNIT: bf16 inputs, whose v_descale is 1.
template <int D, int NT, bool UNIT>
__device__ __forceinline__ void store_output(const PrefillParams& p, const f32x16 (&A)[NT],
                                             float M, float L, int dt0, int64_t q_start, int head,
                                             int nrows, int64_t rs, int qrow, int h) {
  const int64_t o_head = (int64_t)q_start * p.hq + head;
  const rsrc_t orr = make_rsrc(static_cast<unsigned char*>(p.o) + o_head * D * 2,
                               extent_bytes(nrows, rs * D * 2, D * 2,
                                            (p.total_q * p.hq - o_head) * D * 2));
  const uint32_t rowoff = (uint32_t)qrow * (uint32_t)(rs * D * 2);
  const RowFinal fin(L, p.v_descale);
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * (dt0 + j) + 8 * q4 + 4 * h;
      const uint32_t w0 = pack_bf16x2(fin.elem<UNIT>(A[j][4 * q4 + 0]),
                                      fin.elem<UNIT>(A[j][4 * q4 + 1]));
      const uint32_t w1 = pack_bf16x2(fin.elem<UNIT>(A[j][4 * q4 + 2]),
                                      fin.elem<UNIT>(A[j][4 * q4 + 3]));
      buf_store8(orr, rowoff + (uint32_t)d * 2u, u32x2{w0, w1});
    }
  if (p.lse != nullptr) {
    const rsrc_t lr = make_rsrc(p.lse + o_head, extent_bytes(nrows, rs * 4, 4,
                                                             (p.total_q * p.hq - o_head) * 4));
    buf_store4(lr, (h || dt0) ? kParked : (uint32_t)qrow * (uint32_t)(rs * 4),
               f32_bits(finalize_lse(M, L)));
  }
}

// Configurations whose monolithic paged kernel spreads single-token sequences
// over workgroups when given a workspace: all but bf16 D = 192, whose four
// waves hold six output tiles each and have no registers left for the chunk
// partial's stores.
template <int D, bool FP8, bool MONO_PAGED>
constexpr bool kSpread = MONO_PAGED && (FP8 || D <= 128);
// Chunks per spread workgroup: a run of four 512-key chunks keeps a spread
// workgroup's setup small against its 32 blocks while a 32768-token row still
// finishes in a sixteenth of its single-tile time (runs of 1, 2 and 8 measured
// the same on the mixed batch).
constexpr int kSpreadRun = 4;

template <int D, bool FP8, int NW, int WPE, bool SPLIT, bool PAGED, bool WIN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void prefill_kernel(const PrefillParams p) {
  using G = Geom<D, FP8>;
  using C = PrefillCfg<D, FP8, NW, PAGED>;
  static_assert(C::kLds <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
  constexpr int NT = G::kDTiles / C::kDSplit;  // output tiles of this wave
  static_assert(G::kDTiles % C::kDSplit == 0, "D splits into whole 32-column tiles");
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::kLds];
  unsigned char* const sQ = smem;
  unsigned char* const sK = smem + C::kKOff;
  unsigned char* const sV = smem + C::kVOff;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5;
  // Work decode.  Workgroup ids are dealt round-robin to the eight XCDs
  // (id % 8), so the head index varies fastest: with Hq a multiple of 8, XCD x
  // owns query heads [x*Hq/8, (x+1)*Hq/8) -- contiguous GQA groups, whose K/V
  // then stay in that XCD's L2 -- and every XCD gets an equal share of every
  // sequence.  Then the batch, then (split) the chunk, then tiles from the last
  // (heaviest under a causal mask) to the first.
  int id = blockIdx.x;
  int head;
  if (p.hq % 8 == 0) {
    const int per = p.hq / 8;
    const int x = id % 8;
    id /= 8;
    head = x * per + id % per;
    id /= per;
  } else {
    head = id % p.hq;
    id /= p.hq;
  }
  int b = id % p.batch;
  // Sequence bounds of this workgroup's sequence, read below unless the sort
  // has them in LDS already.
  bool bounds_lds = false;
  int lds_q0 = 0, lds_q1 = 0, lds_ctx = 0;
  if constexpr (PAGED && !SPLIT) {
    // A mixed batch can hold a decode or short extend whose single tile scans a
    // long context; handed out last, that tile alone would run past everything
    // else.  Sequences are therefore dealt in descending context length (ties by
    // index): the rank-th longest sequence takes this workgroup's batch slot.
    // Which workgroup computes a tile changes no bit of its result.  The query
    // offsets are read beside the context lengths, so the sequence's bounds
    // need no second memory round trip after the sort.
    __shared__ int sCtx[C::kThreads];
    __shared__ int sCuq[C::kThreads];
    __shared__ int sSeq;
    if (p.batch <= C::kThreads) {
      bounds_lds = p.batch < C::kThreads;  // cu_q has batch + 1 entries
      if (tid < p.batch) sCtx[tid] = p.ctx_lens[tid];
      if (bounds_lds && tid <= p.batch) sCuq[tid] = p.cu_q[tid];
      __syncthreads();
      if (tid < p.batch) {
        const int key = sCtx[tid];
        int rank = 0;
        for (int t = 0; t < p.batch; ++t) {
          const int kt = sCtx[t];
          rank += (kt > key || (kt == key && t < tid)) ? 1 : 0;
        }
        if (rank == b) sSeq = tid;
      }
      __syncthreads();
      b = uniform(sSeq);
      if (bounds_lds) {
        lds_q0 = uniform(sCuq[b]);
        lds_q1 = uniform(sCuq[b + 1]);
        lds_ctx = uniform(sCtx[b]);
      }
    }
  }
  id /= p.batch;
  int chunk = 0;
  if constexpr (SPLIT) {
    chunk = id % p.cmax;
    id /= p.cmax;
  }
  const int tile_rev = id;

  const int q_start = bounds_lds ? lds_q0 : uniform(p.cu_q[b]);
  const int lq = (bounds_lds ? lds_q1 : uniform(p.cu_q[b + 1])) - q_start;
  // Keys: packed rows [cu_k[b], cu_k[b+1]), or the first ctx_lens[b] tokens of
  // the sequence's pages (clamped to its page-table row).
  int k_start = 0, lk;
  if constexpr (PAGED) {
    lk = max(0, min(bounds_lds ? lds_ctx : uniform(p.ctx_lens[b]), p.max_pages * 16));
  } else {
    k_start = uniform(p.cu_k[b]);
    lk = uniform(p.cu_k[b + 1]) - k_start;
  }
  if (lq <= 0 || q_start < 0 || k_start < 0) return;
  // A single-token sequence over a paged cache (a decode row) packs the query
  // heads of its kv head into one tile: row r is query head head + r at the
  // sequence's one position, so the group's K/V stream once instead of once
  // per query head.  Every row runs the arithmetic it runs alone (rows are
  // independent), so the bits are those of the unpacked tiles.  The group's
  // first head computes the tile; the others have nothing to do.
  const int grp_size = p.hq / p.hkv;
  const bool pack = PAGED && lq == 1 && grp_size > 1;
  // With a workspace, a single-token sequence may spread its chunks over the
  // workgroup slots of its tile set (query heads of the set times the tile
  // slots of the launch); see the chunk spread below.
  // A group larger than one tile (several tiles per set) keeps the tiles.
  const bool ds_try = kSpread<D, FP8, PAGED && !SPLIT> && lq == 1 && p.ws_cnt != nullptr &&
                      (pack ? grp_size : 1) <= C::kTileRows;
  const int tset = pack ? grp_size : 1;                // query heads per tile set
  const int hsub = head % tset;                        // this workgroup's head in the set
  const int ds_slot = tile_rev * tset + hsub;          // this workgroup's slot in the set
  head -= hsub;  // the tile set's first query head
  const int nrows = pack ? grp_size : lq;  // real rows of this tile set
  const int64_t rs = pack ? 1 : p.hq;      // row stride in head rows
  auto pos = [&](int i) { return pack ? 0 : i; };  // query position of local row i
  const int ntiles = (nrows + C::kTileRows - 1) / C::kTileRows;
  // Tiles of a packed set (a group larger than one tile has several) go to
  // the workgroups of its heads at the first tile slot: the launch sizes its
  // tile slots by query rows, one for a single-token sequence.
  int tile;
  if (ds_try) {
    tile = 0;
  } else if (pack) {
    if (tile_rev != 0 || hsub >= ntiles) return;
    tile = ntiles - 1 - hsub;
  } else {
    tile = ntiles - 1 - tile_rev;
  }
  if (tile < 0) return;
  const int r0 = tile * C::kTileRows;
  const int g = head / grp_size;

  // Visible keys of local query row i: [row_lo(i), row_hi(i)), bounds on the
  // bottom-right diagonal i + koff (causal, and a sliding window's left and
  // right edges).  Both bounds are nondecreasing in i.
  const int koff = lk - lq;
  // Without WIN the window bounds fold away at compile time (no window set).
  const int wl = WIN ? p.window_left : -1, wr = WIN ? p.window_right : -1;
  auto row_lo = [&](int i) { return wl >= 0 ? max(0, i + koff - wl) : 0; };
  auto row_hi = [&](int i) {
    int hi = lk;
    if (p.causal) hi = min(hi, i + koff + 1);
    if (wr >= 0) hi = min(hi, i + koff + wr + 1);
    return max(hi, 0);
  };
  // Key ranges of this tile's real rows.
  const int last = min(r0 + C::kTileRows, nrows) - 1;
  const int kstart = row_lo(pos(r0));    // first key visible to some row
  const int kend = row_hi(pos(last));    // past the last key visible to some row
  const int nblk = kend > kstart ? (kend + kBlockKeys - 1) / kBlockKeys : 0;
  const int blk_first = kend > kstart ? kstart / kBlockKeys : 0;
  int blk_begin = blk_first, blk_end = nblk;
  if constexpr (SPLIT) {
    blk_begin = max(chunk * kBlocksPerChunk, blk_first);
    blk_end = min(chunk * kBlocksPerChunk + kBlocksPerChunk, nblk);
  }
  // Chunk spread.  A single-token sequence (a decode row; the query heads of
  // its group packed in one tile) scans its whole context on one wave, a chain
  // that outlasts the rest of a mixed batch.  With a workspace, its chunks
  // [ds_first, ds_first + ds_chunks) are dealt to the first ds_count slots of
  // its tile set in contiguous runs of about kSpreadRun chunks, each chunk
  // from the empty state as always (the host sizes the launch's tile slots so
  // that every set has enough); every chunk's partial goes to the workspace,
  // and the slot that
  // completes the set's counter folds them in ascending order and finalises
  // the rows.  That is the fold the single tile runs in registers, on the same
  // partials, so the rows keep their bits.  Sets whose chunks would pass the
  // launch's chunk count (a context length above max_context_len) keep the
  // single tile.
  bool dsplit = false;
  int ds_first = 0, ds_chunks = 0, ds_count = 1;
  if constexpr (kSpread<D, FP8, PAGED && !SPLIT>) {
    if (ds_try) {
      const int cf = blk_first / kBlocksPerChunk;
      const int cl = nblk > blk_first ? (nblk + kBlocksPerChunk - 1) / kBlocksPerChunk : cf;
      const int cn = cl - cf;
      const int cnt = min(tset * p.tiles, (cn + kSpreadRun - 1) / kSpreadRun);
      if (cnt > 1 && cl <= p.cmax) {
        if (ds_slot >= cnt) return;
        dsplit = true;
        ds_first = cf;
        ds_chunks = cn;
        ds_count = cnt;
        blk_begin = max(blk_first, (cf + ds_slot * cn / cnt) * kBlocksPerChunk);
        blk_end = min(nblk, (cf + (ds_slot + 1) * cn / cnt) * kBlocksPerChunk);
      } else if (ds_slot != 0) {
        return;
      }
    }
  }

  // Query group (32 rows) and output columns [32 dt0, 32 (dt0 + NT)) of this wave.
  const int qg = wave % C::kQGroups, dt0 = (wave / C::kQGroups) * NT;
  const int qrow = r0 + 32 * qg + (lane & 31);  // local query row of this lane
  const int lo = row_lo(pos(qrow)), hi = row_hi(pos(qrow));
  // Blocks [wblk_first, wblk_end) hold a key visible to some row of this wave;
  // the others are fully masked for all of its rows (a wave whose rows all lie
  // past the sequence has none).  Such a block leaves m and l exactly as they
  // were (alpha = 1, p = 0) and acc up to the sign of a zero element (adding
  // zero products can turn -0 into +0), which the finalize step erases, so the
  // wave skips its arithmetic while still taking part in the staging and the
  // barriers.
  const int wrow0 = r0 + 32 * ((int)uniform(wave) % C::kQGroups);
  const int wrow_last = min(wrow0 + 31, nrows - 1);
  const bool wactive = wrow0 < nrows;
  const int wlo = wactive ? row_lo(pos(wrow0)) : 0;
  const int wlo_max = wactive ? row_lo(pos(wrow_last)) : 0;  // a lower edge masks blocks below it
  const int whi = wactive ? row_hi(pos(wrow_last)) : 0;
  const int whi_min = wactive ? row_hi(pos(wrow0)) : 0;  // an upper edge masks blocks past it
  // Bounds of the unmasked class: this wave's for sliding windows and paged
  // caches; the tile's (every row of the tile sees the block) for contiguous
  // causal tiles, where the per-wave class measured slower.  A fully visible
  // block gives the same bits in either class.
  const int mlo = (WIN || PAGED) ? wlo_max : row_lo(pos(last));
  const int mhi = (WIN || PAGED) ? whi_min : row_hi(pos(r0));
  const int wblk_first = wlo / kBlockKeys;
  const int wblk_end = whi > wlo ? (whi + kBlockKeys - 1) / kBlockKeys : 0;
  auto wave_live = [&](int blk) { return blk >= wblk_first && blk < wblk_end; };

  if constexpr (SPLIT) {
    if (blk_begin >= blk_end) {
      // Empty chunk for this tile: every row's partial is (m, l) = (-inf, 0).
      const int64_t ml_head = ((int64_t)chunk * p.total_q + q_start) * p.hq + head;
      const rsrc_t mlr = make_rsrc(p.part_ml + 2 * ml_head,
                                   extent_bytes(nrows, rs * 8, 8,
                                                ((int64_t)(chunk + 1) * p.total_q * p.hq - ml_head) * 8));
      const uint32_t off = h ? kParked : (uint32_t)qrow * (uint32_t)(rs * 8);
      buf_store8(mlr, off, u32x2{f32_bits(-INFINITY), 0u});
      return;
    }
  }

  if constexpr (C::kPairPC) {
    // Score/PV pair schedule (e4m3 wide heads from packed rows).  Waves w and
    // w + 4 share a SIMD and the 32 query rows of group qg = w % 4.  The score
    // wave computes S_j = K_j Q^T and the softmax update of block j once, for
    // both, and publishes P_j^T and (alpha_j, m_j, l_j) in P slot j % 2.  Step j
    // runs the softmax of block j, issues S_{j+1} on the matrix cores first so
    // that it overlaps that softmax, and applies block j - 1 to the output: the
    // score wave to tiles [0, kPairTilesS), the PV wave, which reads P_{j-1} from
    // its slot, to the other kPairTilesV.  The PV waves do all the staging
    // through registers, in two register sets used on alternate steps: step j
    // loads K_{j+3} and V_{j+1} into set (j+1) % 2, issues its P V of block
    // j - 1, then writes K_{j+2} into K stage (j+2) % 3 and V_j, widened to
    // bf16, into V stage j % 2 from set j % 2 (loaded in step j - 1, so a load
    // has a whole step to arrive).  The widening comes after the P V MFMAs so
    // that it runs under them, beside the score wave's softmax, and the
    // SIMD's matrix work is not all at the start and end of the step (writing
    // the stages first was 2.5% slower).
    // Slot use in step j: K stage (j+1) % 3 is read (written in step j - 1) and
    // K stage (j+2) % 3 written (last read in step j - 2); V stage (j-1) % 2 read
    // (written in step j - 1), V stage j % 2 written (last read in step j - 1);
    // P slot (j-1) % 2 read (written in step j - 1), P slot j % 2 written (last
    // read in step j - 1).  One barrier per step, which completes the step's
    // LDS writes but leaves its loads in flight (barrier_lds).  The step loop is
    // unrolled by two so that the register sets are fixed in the code.  Every
    // operand reaches the same MFMA and VALU operations as in the other
    // schedules, so the bits are the same.
    constexpr int NTS = C::kPairTilesS, NTV = C::kPairTilesV;
    constexpr int kChunks = kBlockKeys * G::kChunks16;  // 16-byte chunks of a K or V block
    constexpr int kPer = (kChunks + 255) / 256;          // per PV-wave thread
    const int wv = uniform(wave);
    const bool score = wv < 4;
    const int qgp = wv & 3;
    const int dtp = score ? 0 : NTS;  // first output tile of this wave
    unsigned char* const sKp = smem + C::kPcKOff;
    unsigned char* const sVp = smem + C::kPcVOff;
    unsigned char* const sP = smem + C::kPcPOff;
    auto pslot = [&](int j) { return sP + ((j & 1) * C::kQGroups + qgp) * C::kPSlot; };
    auto kstage = [&](int j) { return sKp + (j % C::kPcKStages) * C::kKStage; };
    const float c = p.c_scale;
    // The two roles run separate instantiations of the step loop, so each
    // holds only its own accumulators and running totals in registers.
    auto run_role = [&](auto role) {
      constexpr bool S = decltype(role)::value;
      constexpr int NTX = S ? NTS : NTV;
      float m = -INFINITY, l = 0.0f, M = -INFINITY, L = 0.0f;
      f32x16 acc[NTX], A[NTX];
#pragma unroll
      for (int t = 0; t < NTX; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = A[t][i] = 0.0f;
      auto softmax = [&](int blk, const f32x16 (&s)[2], float& alpha, u32x4 (&pb)[4]) {
        const int b0 = kBlockKeys * blk;
        if (b0 >= mlo && b0 + kBlockKeys <= mhi) {
          softmax_block<kNoMask>(s, h, c, 0, 0, m, l, alpha, pb);
        } else if (b0 >= wlo_max) {
          softmax_block<kMaskHi>(s, h, c, 0, hi - b0, m, l, alpha, pb);
        } else {
          softmax_block<kMaskLoHi>(s, h, c, lo - b0, hi - b0, m, l, alpha, pb);
        }
      };
      // The fold of a finished chunk into the running total (the function
      // every schedule runs); the accumulator restarts from +0.
      auto fold = [&](float mc, float lc) {
        float ca, cb;
        bool keep;
        merge_stats(M, L, mc, lc, ca, cb, keep);
#pragma unroll
        for (int t = 0; t < NTX; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            A[t][i] = merge_elem(A[t][i], acc[t][i], keep, ca, cb);
            acc[t][i] = 0.0f;
          }
      };
      if (blk_begin < blk_end) {
        const int n = blk_end - blk_begin;
        const int64_t q_head = (int64_t)q_start * p.hq + head;
        const int64_t kv_head = (int64_t)k_start * p.hkv + g;
        const uint32_t q_row_bytes = (uint32_t)(rs * G::kRowBytes);
        const uint32_t kv_row_bytes = (uint32_t)(p.hkv * G::kRowBytes);
        const unsigned char* qb = static_cast<const unsigned char*>(p.q) + q_head * G::kRowBytes;
        const unsigned char* kb = static_cast<const unsigned char*>(p.k) + kv_head * G::kRowBytes;
        const unsigned char* vb = static_cast<const unsigned char*>(p.v) + kv_head * G::kRowBytes;
        // Window-sized K/V descriptors over key rows [kstart, kend).
        const uint32_t kv_ext =
            extent_bytes(kend - kstart, kv_row_bytes, G::kRowBytes,
                         (p.total_k * p.hkv - kv_head) * G::kRowBytes - (int64_t)kstart * kv_row_bytes);
        const int64_t kv_win = (int64_t)kstart * kv_row_bytes;
        const rsrc_t kr = make_rsrc(kb + kv_win, kv_ext);
        const rsrc_t vr = make_rsrc(vb + kv_win, kv_ext);
        if constexpr (S) {
          // Score wave: its lane's Q^T operands straight from HBM (rows past
          // the sequence read as zeros), S_0, then the step loop.
          const rsrc_t qr = make_rsrc(qb, extent_bytes(nrows, q_row_bytes, G::kRowBytes,
                                                       (p.total_q * p.hq - q_head) * G::kRowBytes));
          QOperands<D, true> qop;
          const uint32_t qoff = (uint32_t)(r0 + 32 * qgp + (lane & 31)) * q_row_bytes;
#pragma unroll
          for (int st = 0; st < QOperands<D, true>::kCount; ++st)
            qop.q[st] = buf_load16(qr, qoff + (uint32_t)(64 * (st >> 1) + 32 * h + 16 * (st & 1)));
          wait_vm();
          __syncthreads();  // K_0 and K_1 are in their stages
          f32x16 sc[2][2];  // scores of blocks j (set j % 2) and j + 1
          if (wave_live(blk_begin)) qk_scores_qreg<D, true, C::kKPage>(sc[0], qop, kstage(0), lane);
          u32x4 pb_prev[4] = {};
          float alpha_prev = 1.0f;
          auto step = [&](int j, auto set) {
            constexpr int X = decltype(set)::value;
            const int blk = blk_begin + j;
            // Block j - 1 is the last block of its chunk (or of the range).
            const bool chunk_end = j > 0 && (blk % kBlocksPerChunk == 0 || j == n);
            const float mc = m, lc = l;
            if (chunk_end && j < n) {  // block j opens a new chunk from the empty state
              m = -INFINITY;
              l = 0.0f;
            }
            if (j + 1 < n && wave_live(blk + 1))
              qk_scores_qreg<D, true, C::kKPage>(sc[X ^ 1], qop, kstage(j + 1), lane);
            u32x4 pb[4];
            float alpha = 1.0f;
            if (j < n && wave_live(blk)) {
              softmax(blk, sc[X], alpha, pb);
              unsigned char* const ps = pslot(j);
#pragma unroll
              for (int k = 0; k < 4; ++k) lds_store16(ps, (uint32_t)(k * C::kPRow + lane * 16), pb[k]);
              if (h == 0)
                lds_store16(ps, (uint32_t)(4 * C::kPRow + lane * 16),
                            u32x4{f32_bits(alpha), f32_bits(m), f32_bits(l), 0u});
            }
            if (j > 0 && wave_live(blk - 1)) {
              rescale_acc<NTX>(acc, alpha_prev);
              pv_mfma<D, NTX>(acc, 0, pb_prev, sVp + ((j - 1) & 1) * C::kVStage, lane);
            }
            if constexpr (!SPLIT) {
              if (chunk_end) fold(mc, lc);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) pb_prev[k] = pb[k];
            alpha_prev = alpha;
            barrier_lds();
          };
          int j = 0;
          for (; j + 1 <= n; j += 2) {
            step(j, std::integral_constant<int, 0>{});
            step(j + 1, std::integral_constant<int, 1>{});
          }
          if (j <= n) step(j, std::integral_constant<int, 0>{});
        } else {
          // PV wave: K and V through registers (two sets), K two blocks
          // ahead of its use and V one.
          const int vt = tid - 256;  // PV-wave thread index
          u32x4 kreg[2][kPer], vreg[2][kPer];
          auto load = [&](const rsrc_t& r, int blk, u32x4 (&dst)[kPer]) {
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
              const int x = vt + 256 * u;
              if (kPer * 256 == kChunks || x < kChunks) {
                const int rr = x / G::kChunks16, col = x % G::kChunks16;
                dst[u] = buf_load16(r, (uint32_t)((int64_t)(blk * kBlockKeys - kstart + rr) * kv_row_bytes) +
                                           (uint32_t)col * 16u);
              }
            }
          };
          auto k_store = [&](unsigned char* ks, const u32x4 (&src)[kPer]) {
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
              const int x = vt + 256 * u;
              if (kPer * 256 == kChunks || x < kChunks) {
                const int rr = x / G::kChunks16, col = x % G::kChunks16;
                lds_store16(ks, (uint32_t)(rr * G::kKRow + col * 16), src[u]);
              }
            }
          };
          auto v_store = [&](unsigned char* vs, const u32x4 (&src)[kPer]) {
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
              const int x = vt + 256 * u;
              if (kPer * 256 == kChunks || x < kChunks) {
                const int rr = x / G::kChunks16, col = x % G::kChunks16;
                const u32x2 a = e4m3x4_to_bf16x4(src[u][0]), b2 = e4m3x4_to_bf16x4(src[u][1]);
                const u32x2 c2 = e4m3x4_to_bf16x4(src[u][2]), d2 = e4m3x4_to_bf16x4(src[u][3]);
                const uint32_t o = (uint32_t)(rr * G::kVRow + col * 32);
                lds_store16(vs, o, u32x4{a[0], a[1], b2[0], b2[1]});
                lds_store16(vs, o + 16, u32x4{c2[0], c2[1], d2[0], d2[1]});
              }
            }
          };
          // Prologue: K_0 and K_1 into their stages; K_2 and V_0 into set 0.
          load(kr, blk_begin, kreg[0]);
          load(kr, blk_begin + 1, kreg[1]);
          k_store(kstage(0), kreg[0]);
          k_store(kstage(1), kreg[1]);
          load(kr, blk_begin + 2, kreg[0]);
          load(vr, blk_begin, vreg[0]);
          wait_vm();
          __syncthreads();  // K_0 and K_1 are in their stages
          auto step = [&](int j, auto set) {
            constexpr int X = decltype(set)::value;
            const int blk = blk_begin + j;
            const bool chunk_end = j > 0 && (blk % kBlocksPerChunk == 0 || j == n);
            // Loads of this step into the other set, then the stores of the
            // blocks loaded in the previous step.  They run in every step, also
            // past the last block (rows past the descriptors read as zeros, and
            // those stages are not read in this step), so that every step has
            // the same count of loads in flight and the waits before the stores
            // leave this step's loads outstanding.
            load(kr, blk + 3, kreg[X ^ 1]);
            load(vr, blk + 1, vreg[X ^ 1]);
            if (j > 0 && wave_live(blk - 1)) {
              const unsigned char* const ps = pslot(j - 1);
              u32x4 pb[4];
#pragma unroll
              for (int k = 0; k < 4; ++k) pb[k] = lds_load16(ps, (uint32_t)(k * C::kPRow + lane * 16));
              const u32x4 st = lds_load16(ps, (uint32_t)(4 * C::kPRow + (lane & 31) * 16));
              m = bits_f32(st[1]);
              l = bits_f32(st[2]);
              rescale_acc<NTX>(acc, bits_f32(st[0]));
              pv_mfma<D, NTX>(acc, NTS, pb, sVp + (X ^ 1) * C::kVStage, lane);
            }
            k_store(kstage(j + 2), kreg[X]);
            v_store(sVp + X * C::kVStage, vreg[X]);
            if constexpr (!SPLIT) {
              if (chunk_end) {
                fold(m, l);
                m = -INFINITY;
                l = 0.0f;
              }
            }
            barrier_lds();
          };
          int j = 0;
          for (; j + 1 <= n; j += 2) {
            step(j, std::integral_constant<int, 0>{});
            step(j + 1, std::integral_constant<int, 1>{});
          }
          if (j <= n) step(j, std::integral_constant<int, 0>{});
          wait_vm();  // nothing is left in flight past the loop
        }
      }
      // Epilogue: each wave stores its own output tiles.
      if constexpr (SPLIT) {
        store_partial<D, NTX>(p, acc, m, l, dtp, chunk, q_start, head, nrows, rs, qrow, h);
      } else {
        store_output<D, NTX, !FP8>(p, A, M, L, dtp, q_start, head, nrows, rs, qrow, h);
      }
    };
    if (score) {
      run_role(std::true_type{});
    } else {
      run_role(std::false_type{});
    }
    return;
  }

  const float c = p.c_scale;
  f32x16 acc[NT];
  f32x16 A[NT];
  float m = -INFINITY, l = 0.0f, M = -INFINITY, L = 0.0f;
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[j][i] = 0.0f;
      A[j][i] = 0.0f;
    }
  // Softmax update of block blk, masked according to its class: no mask where
  // every row (of the wave, or of the tile) sees all 64 keys, the upper edge
  // alone where no row of the wave has its lower edge inside the block, both
  // edges otherwise (the three give the same bits wherever a key is visible).
  auto softmax = [&](int blk, const f32x16 (&s)[2], float& alpha, u32x4 (&pb)[4]) {
    const int b0 = kBlockKeys * blk;
    if (b0 >= mlo && b0 + kBlockKeys <= mhi) {
      softmax_block<kNoMask>(s, h, c, 0, 0, m, l, alpha, pb);
    } else if (b0 >= wlo_max) {
      softmax_block<kMaskHi>(s, h, c, 0, hi - b0, m, l, alpha, pb);
    } else {
      softmax_block<kMaskLoHi>(s, h, c, lo - b0, hi - b0, m, l, alpha, pb);
    }
  };

  // The end of a chunk folds its partial into the running total, or, when
  // the chunk spread deals this tile set's chunks out (SP), stores the partial
  // in the workspace (the wave's rows and output tiles; one lane per row for
  // (m, l)).  The accumulator restarts from +0 either way.
  auto fold_chunk = [&]() {
    float ca, cb;
    bool keep;
    merge_stats(M, L, m, l, ca, cb, keep);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        A[t][i] = merge_elem(A[t][i], acc[t][i], keep, ca, cb);
        acc[t][i] = 0.0f;
      }
    m = -INFINITY;
    l = 0.0f;
  };
  auto store_chunk = [&](int c) {
    const int64_t slot = ((int64_t)c * p.batch + b) * p.hq + head;
    const rsrc_t mlr = make_rsrc(p.ws_ml + 2 * slot, (uint32_t)nrows * 8u);
    buf_store8(mlr, (h || dt0) ? kParked : (uint32_t)qrow * 8u, u32x2{f32_bits(m), f32_bits(l)});
    const rsrc_t ar = make_rsrc(p.ws_acc + slot * D, (uint32_t)nrows * D * 4u);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * (dt0 + t) + 8 * q4 + 4 * h;
        buf_store16(ar, (uint32_t)(qrow * D + d) * 4u,
                    u32x4{f32_bits(acc[t][4 * q4 + 0]), f32_bits(acc[t][4 * q4 + 1]),
                          f32_bits(acc[t][4 * q4 + 2]), f32_bits(acc[t][4 * q4 + 3])});
        for (int i = 0; i < 4; ++i) acc[t][4 * q4 + i] = 0.0f;
      }
    m = -INFINITY;
    l = 0.0f;
  };

  // The block loop, instantiated twice where the chunk spread exists: the
  // copy that stores chunk partials (SP) runs only on spread tiles, so the
  // registers of the ordinary copy are those of a kernel without the spread.
  auto run_blocks = [&](auto sp_tag) {
  constexpr bool SP = decltype(sp_tag)::value;
  auto end_chunk = [&](int cidx) {
    if constexpr (SP) {
      store_chunk(cidx);
    } else {
      fold_chunk();
    }
  };
  if (blk_begin < blk_end) {
    const int64_t q_head = (int64_t)q_start * p.hq + head;
    const int64_t kv_head = (int64_t)k_start * p.hkv + g;
    const uint32_t q_row_bytes = (uint32_t)(rs * G::kRowBytes);
    const uint32_t kv_row_bytes = (uint32_t)(p.hkv * G::kRowBytes);
    const unsigned char* qb = static_cast<const unsigned char*>(p.q) + q_head * G::kRowBytes;
    const unsigned char* kb = static_cast<const unsigned char*>(p.k) + kv_head * G::kRowBytes;
    const unsigned char* vb = static_cast<const unsigned char*>(p.v) + kv_head * G::kRowBytes;
    const rsrc_t qr = make_rsrc(qb, extent_bytes(nrows, q_row_bytes, G::kRowBytes,
                                                 (p.total_q * p.hq - q_head) * G::kRowBytes));
    // Window-sized K/V descriptors: they cover key rows [kstart, kend) of the
    // sequence, the keys some row of this tile can see (aiter MQA-logits page:
    // num_records is the window test), so keys outside read as zeros.
    const uint32_t kv_ext =
        extent_bytes(kend - kstart, kv_row_bytes, G::kRowBytes,
                     (p.total_k * p.hkv - kv_head) * G::kRowBytes - (int64_t)kstart * kv_row_bytes);
    const int64_t kv_win = (int64_t)kstart * kv_row_bytes;
    const rsrc_t kr = make_rsrc(kb + (PAGED ? 0 : kv_win), PAGED ? 0u : kv_ext);
    const rsrc_t vr = make_rsrc(vb + (PAGED ? 0 : kv_win), PAGED ? 0u : kv_ext);
    // Paged caches: the kv head's slot-0 offset of a page, -1 outside the cache.
    const int32_t* const table = PAGED ? p.page_table + (int64_t)b * p.max_pages : nullptr;
    auto page_base = [&](int j) -> int64_t {
      const int64_t pg = table[j / 16];
      return (pg >= 0 && pg < p.num_pages) ? pg * p.page_stride + (int64_t)g * p.head_stride : -1;
    };
    const int wv = uniform(wave);
    // The direct stager of this sequence's keys (packed rows or cache pages).
    auto make_direct = [&]() {
      if constexpr (C::kDirectK) {
        DirectStager<D, NW, true> st;  // K only
        st.init(wv, lane, kr, vr, kv_row_bytes, kstart);
        return st;
      } else if constexpr (!C::kDirect) {
        return 0;  // staged through registers
      } else if constexpr (PAGED) {
        PagedDirectStager<D, NW, C::kKPage> st;
        const int64_t head_off = (int64_t)g * p.head_stride * G::kEs;
        st.init(wv, lane, static_cast<const unsigned char*>(p.k) + head_off,
                static_cast<const unsigned char*>(p.v) + head_off, table, p.num_pages,
                p.page_stride * G::kEs, (uint32_t)(p.token_stride * G::kEs), lk, p.max_pages);
        return st;
      } else {
        DirectStager<D, NW> st;
        st.init(wv, lane, kr, vr, kv_row_bytes, kstart);
        return st;
      }
    };

    if constexpr (C::kDirect && NW == 8) {
    if constexpr (SP) {
    // Spread tiles of a single-token sequence (bf16 paged caches).  Only the
    // waves holding the tile's rows compute (one wave for a kv group of up to
    // 32 query heads), and with no second wave of the SIMD to share the work
    // there is nothing to ping-pong: a block's loads have only one wave's
    // block of arithmetic to hide under.  So the blocks go
    // through three K/V stages, the third at the end of the Q tile's region
    // (whose start keeps the Q rows of up to kDeepRows rows; the waves read
    // their Q^T operands from LDS, which keeps their registers at what the
    // ping-pong needs), and step j issues the loads of block j+2 from inline
    // assembly, so they stay in flight while the step computes block j; the
    // step ends by waiting for block j+1's loads (a staging wave's loads of
    // block j+2 may stay outstanding) and a barrier that leaves them in flight.
    // Block b lives in stage b % 3 (blocks relative to blk_begin) and is
    // written in step b - 2, after the barrier that ended step b - 3, the last
    // reads of that stage.  A tile with more rows uses two stages, one block
    // ahead.  The page-table entries of the run arrive in one vector load at
    // the start and reach the loads by readlane, so no table load sits behind
    // staging loads in the in-order wait.  Each block's arithmetic is the one
    // every schedule runs (scores, softmax update, rescale, P V), so the bits
    // are the same.
    constexpr int kSt2 = C::kQBytes - C::kKStage - C::kVStage;  // third stage, K then V
    constexpr int kDeepRows = kSt2 / G::kQRow / 32 * 32;
    static_assert(kDeepRows >= 32, "the third stage leaves room for one wave's Q rows");
    const int n = blk_end - blk_begin;
    const bool deep = nrows <= kDeepRows;
    const int ns = deep ? 3 : 2;  // stages, and blocks in flight plus one
    // The second half of the waves stage, one cache page each (a wave that
    // computes a block while its own LDS-destination loads are outstanding
    // ran 8% slower); the first half computes (only groups of more than 128
    // rows compute on the second half too).  The stager takes a copy of the
    // lane index that the compiler cannot identify with lane, so its per-lane
    // offsets are computed here and not hoisted above the branch into a live
    // range shared with the ping-pong's stager.  (Its wave count is spelled
    // through SP so that kernels without the spread never instantiate it.)
    constexpr int kStageWaves = SP ? NW / 2 : NW;
    int lane_x = lane;
    asm volatile("" : "+v"(lane_x));
    PagedDirectStager<D, kStageWaves, C::kKPage> dst;
    {
      const int64_t head_off = (int64_t)g * p.head_stride * G::kEs;
      dst.init(wv % kStageWaves, lane_x, static_cast<const unsigned char*>(p.k) + head_off,
               static_cast<const unsigned char*>(p.v) + head_off, table, p.num_pages,
               p.page_stride * G::kEs, (uint32_t)(p.token_stride * G::kEs), lk, p.max_pages);
    }
    using St = decltype(dst);
    static_assert(St::kWavesPerPage == 1, "one staging wave per page region");
    const bool stager = wv >= NW - kStageWaves;
    constexpr int kLoads = St::loads_per_block(0);  // per staging wave and block
    auto kst = [&](int sidx) { return sidx == 2 ? sQ + kSt2 : sK + sidx * C::kKStage; };
    auto vst = [&](int sidx) { return sidx == 2 ? sQ + kSt2 + C::kKStage : sV + sidx * C::kVStage; };
    int ebase = blk_begin;
    int32_t ent = dst.entries(ebase, lane);
    // Scalar table entry of block blk (blocks in increasing order); a run past
    // 64 blocks reloads the entries, waiting for them at once, so that no wait
    // for them remains on the path of the steps that follow.
    auto entry = [&](int blk) {
      if (blk - ebase >= kWave) {
        ebase = blk;
        ent = dst.entries(ebase, lane);
        asm volatile("" ::"v"(ent));
      }
      return __builtin_amdgcn_readlane(ent, blk - ebase);
    };
    for (int b = 0; b < ns - 1 && b < n; ++b) {
      dst.use_entry(entry(blk_begin + b));
      if (stager) {
        dst.issue_k(blk_begin + b, kst(b), wv);
        dst.issue_v(blk_begin + b, vst(b), wv);
      }
    }
    for (int x = tid; x < C::kTileRows * G::kChunks16; x += C::kThreads) {
      const int r = x / G::kChunks16, col = x % G::kChunks16;
      if (!deep || r < kDeepRows)
        lds_store16(sQ, (uint32_t)(r * G::kQRow + col * 16),
                    buf_load16(qr, (uint32_t)(r0 + r) * q_row_bytes + (uint32_t)col * 16u));
    }
    wait_vm();
    __syncthreads();
    const unsigned char* const sQw = sQ + (32 * qg) * G::kQRow;
    int cur = 0;  // stage of block j; block j + ns - 1 goes to the stage before it
    for (int j = 0; j < n; ++j) {
      const int blk = blk_begin + j;
      const int ahead_st = cur == 0 ? ns - 1 : cur - 1;
      const bool ahead = j + ns - 1 < n;
      if (ahead && stager) {
        dst.use_entry(entry(blk + ns - 1));
        dst.template issue_k<true>(blk + ns - 1, kst(ahead_st), wv);
        dst.template issue_v<true>(blk + ns - 1, vst(ahead_st), wv);
      }
      if (wave_live(blk)) {
        f32x16 s[2];
        qk_scores_qlds<D, FP8, C::kKPage>(s, sQw, kst(cur), lane);
        float alpha;
        u32x4 pb[4];
        softmax(blk, s, alpha, pb);
        pv_accumulate<D, NT>(acc, dt0, alpha, pb, vst(cur), lane);
      }
      if ((blk + 1) % kBlocksPerChunk == 0 || blk + 1 == blk_end) end_chunk(blk / kBlocksPerChunk);
      // Block j+1 has landed; with three stages a staging wave's loads of
      // block j+2 (issued last) may stay outstanding.
      if (ahead && deep && stager) {
        wait_vm_n<kLoads>();
      } else {
        wait_vm();
      }
      barrier_lds();
      cur = cur == ns - 1 ? 0 : cur + 1;
    }
    } else {
    // Ping-pong (bf16 staged directly, two waves per SIMD).  Each wave
    // alternates an MFMA phase (P V of block j-1, then S_j = K_j Q^T) and a
    // VALU phase (the softmax update of block j and the rescale of acc), one
    // barrier after each.  The second half of the waves (w >= NW/2, which
    // shares SIMDs with the first half: wave w and w+4 sit on one SIMD) runs
    // one phase behind -- one extra barrier at the start, the first half one
    // at the end -- so each SIMD holds one wave of each phase.
    //
    // Staging event e loads K block e+1 into K stage (e+1)%2 and V block e
    // into V stage e%2 (blocks relative to blk_begin), each wave its own
    // segments.  The first half performs event j in its VALU phase j, the
    // second half event j+1 (events up to the lag in the prologue); a wave's
    // loads land before the barrier that ends the phase that issued them.
    // In barrier slots (first half: MFMA phase j = slot 2j, VALU phase j =
    // slot 2j+1; second half one slot later), K_j is read in slots 2j, 2j+1
    // and written in slots 2j-2, 2j-1; V_j is read in 2j+2, 2j+3 and written
    // in 2j, 2j+1: every write falls after the last read of the block two
    // earlier in the same stage and before the first read of its own block.
    const int n = blk_end - blk_begin;
    const int lag = wv >= NW / 2 ? 1 : 0;
    auto dst = make_direct();
    // event e: K block e+1 -> K stage (e+1)&1, V block e -> V stage e&1 (relative
    // blocks).  A wave's events run in order, so after issuing event e it looks
    // up (paged caches) the blocks of event e+1.
    dst.prefetch(blk_begin, blk_begin - 1);
    auto event = [&](int e) {
      dst.latch();
      if (e + 1 < n) dst.issue_k(blk_begin + e + 1, sK + ((e + 1) & 1) * C::kKStage, wv);
      if (e >= 0 && e < n) dst.issue_v(blk_begin + e, sV + (e & 1) * C::kVStage, wv);
      dst.prefetch(blk_begin + e + 2, blk_begin + e + 1);
    };
    event(-1);
    if (lag) event(0);
    for (int x = tid; x < C::kTileRows * G::kChunks16; x += C::kThreads) {
      const int r = x / G::kChunks16, col = x % G::kChunks16;
      lds_store16(sQ, (uint32_t)(r * G::kQRow + col * 16),
                  buf_load16(qr, (uint32_t)(r0 + r) * q_row_bytes + (uint32_t)col * 16u));
    }
    wait_vm();
    __syncthreads();
    if (lag) __syncthreads();
    const unsigned char* const sQw = sQ + (32 * qg) * G::kQRow;
    // bf16 from packed rows: the wave's Q^T operands move from the LDS tile to
    // registers once.  Over a paged cache they are read from the tile every
    // block, which leaves the registers that the paged staging holds.
    QOperands<D, FP8> qop;
    if constexpr (!FP8 && !PAGED) qop.load(sQw + (lane & 31) * G::kQRow, lane);
    u32x4 pb[4];
    for (int j = 0; j < n; ++j) {
      const int blk = blk_begin + j;
      const bool live = wave_live(blk);  // this wave computes block j
      __builtin_amdgcn_s_setprio(2);  // MFMA phase ahead of the other half's VALU
      if (j > 0) {
        if (wave_live(blk - 1)) pv_mfma<D, NT>(acc, dt0, pb, sV + ((j - 1) & 1) * C::kVStage, lane);
      }
      f32x16 s[2];
      if (live) {
        if constexpr (FP8 || PAGED) {
          qk_scores_qlds<D, FP8, C::kKPage>(s, sQw, sK + (j & 1) * C::kKStage, lane);
        } else {
          qk_scores_qreg<D, FP8, C::kKPage>(s, qop, sK + (j & 1) * C::kKStage, lane);
        }
      }
      if constexpr (!SPLIT) {
        if (j > 0 && blk % kBlocksPerChunk == 0) end_chunk(blk / kBlocksPerChunk - 1);
      }
      __syncthreads();
      __builtin_amdgcn_s_setprio(0);
      event(j + lag);
      if (live) {
        float alpha;
        softmax(blk, s, alpha, pb);
        rescale_acc<NT>(acc, alpha);
      }
      wait_vm();
      __syncthreads();
    }
    if (wave_live(blk_end - 1)) pv_mfma<D, NT>(acc, dt0, pb, sV + ((n - 1) & 1) * C::kVStage, lane);
    if constexpr (!SPLIT) end_chunk((blk_end - 1) / kBlocksPerChunk);
    if (!lag) __syncthreads();
    }
      } else {
    const int n = blk_end - blk_begin;
    KVStager<D, FP8, NW> rst;
    // Register staging of block blk: K and V, or V alone where K is loaded
    // directly (kDirectK); the direct K load of a block is issued before its V
    // loads, so the wait for V covers it.
    auto reg_load = [&](int blk) {
      if constexpr (PAGED) {
        rst.load_paged(static_cast<const unsigned char*>(p.k), static_cast<const unsigned char*>(p.v),
                       blk * kBlockKeys, lk, p.token_stride, page_base, tid);
      } else {
        rst.load(kr, blk * kBlockKeys - kstart, !C::kDirectK, vr, blk * kBlockKeys - kstart, true,
                 kv_row_bytes, tid);
      }
    };
    auto dst = make_direct();
    if constexpr (C::kDirect) {
      dst.prefetch(blk_begin, blk_begin);
      dst.latch();
      dst.issue_k(blk_begin, sK, wv);
      dst.issue_v(blk_begin, sV, wv);
    } else {
      if constexpr (C::kDirectK) dst.issue_k(blk_begin, sK, wv);
      reg_load(blk_begin);
    }
    // Q tile -> LDS (rows past the sequence read as zero).
    for (int x = tid; x < C::kTileRows * G::kChunks16; x += C::kThreads) {
      const int r = x / G::kChunks16, col = x % G::kChunks16;
      lds_store16(sQ, (uint32_t)(r * G::kQRow + col * 16),
                  buf_load16(qr, (uint32_t)(r0 + r) * q_row_bytes + (uint32_t)col * 16u));
    }
    if constexpr (C::kDirect) {
      wait_vm();
    } else {
      rst.store(sK, !C::kDirectK, sV, true, tid);
      if constexpr (C::kDirectK) wait_vm();
    }
    __syncthreads();

    const unsigned char* const sQw = sQ + (32 * qg) * G::kQRow;  // this wave's Q rows
    // e4m3 from packed rows (K staged directly, registers to spare): the
    // wave's Q^T operands move from the LDS tile to registers once.
    QOperands<D, FP8> qop;
    if constexpr (C::kDirectK) qop.load(sQw + (lane & 31) * G::kQRow, lane);
    for (int j = 0; j < n; ++j) {
      const int blk = blk_begin + j, cur = j & 1;
      const bool more = j + 1 < n;
      // Block j+1 into the other stage; its previous block was retired by the
      // barrier that ended block j-1.
      if (more) {
        if constexpr (C::kDirect) {
          dst.prefetch(blk + 1, blk + 1);
          dst.latch();
          dst.issue_k(blk + 1, sK + (cur ^ 1) * C::kKStage, wv);
          dst.issue_v(blk + 1, sV + (cur ^ 1) * C::kVStage, wv);
        } else {
          if constexpr (C::kDirectK) dst.issue_k(blk + 1, sK + (cur ^ 1) * C::kKStage, wv);
          reg_load(blk + 1);
        }
      }
      if (wave_live(blk)) {
        f32x16 s[2];
        if constexpr (C::kDirectK) {
          qk_scores_qreg<D, FP8, C::kKPage>(s, qop, sK + cur * C::kKStage, lane);
        } else {
          qk_scores_qlds<D, FP8, C::kKPage>(s, sQw, sK + cur * C::kKStage, lane);
        }
        float alpha;
        u32x4 pb[4];
        softmax(blk, s, alpha, pb);
        pv_accumulate<D, NT>(acc, dt0, alpha, pb, sV + cur * C::kVStage, lane);
      }
      if constexpr (!SPLIT) {
        if ((blk + 1) % kBlocksPerChunk == 0 || blk + 1 == blk_end) end_chunk(blk / kBlocksPerChunk);
      }
      if (more) {
        if constexpr (C::kDirect) {
          wait_vm();
        } else {
          rst.store(sK + (cur ^ 1) * C::kKStage, !C::kDirectK, sV + (cur ^ 1) * C::kVStage, true,
                    tid);
          if constexpr (C::kDirectK) wait_vm();
        }
      }
      __syncthreads();
    }
      }
  }
  };
  if constexpr (kSpread<D, FP8, PAGED && !SPLIT>) {
    if (dsplit) {
      run_blocks(std::true_type{});
      // Count this workgroup in (its partial stores made visible at device
      // scope first); the one that completes the set's count folds every chunk
      // partial in ascending order, finalises the rows and clears the counter
      // for the next launch.
      __shared__ int sLast;
      __syncthreads();
      int32_t* const cnt = p.ws_cnt + (int64_t)b * p.hkv + g;
      if (tid == 0) {
        __threadfence();
        const int done = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        sLast = done == ds_count - 1 ? 1 : 0;
        if (sLast) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (!sLast) return;
      __threadfence();
      const int64_t o_head = (int64_t)q_start * p.hq + head;
      const rsrc_t orr = make_rsrc(static_cast<unsigned char*>(p.o) + o_head * D * 2,
                                   (uint32_t)nrows * D * 2u);
      const rsrc_t lr = make_rsrc(p.lse != nullptr ? p.lse + o_head : nullptr,
                                  p.lse != nullptr ? (uint32_t)nrows * 4u : 0u);
      // The partials are read kBatch chunks at a time (all loads issued before
      // the first fold), so the fold waits on one memory round trip per batch.
      constexpr int kBatch = 16;
      const int cend = ds_first + ds_chunks;
      for (int e = tid; e < nrows * D; e += C::kThreads) {
        const int r = e / D, d = e % D;
        float Mx = -INFINITY, Lx = 0.0f, Ax = 0.0f;
        for (int c0 = ds_first; c0 < cend; c0 += kBatch) {
          float mv[kBatch], lv[kBatch], av[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const int64_t slot = ((int64_t)min(c0 + u, cend - 1) * p.batch + b) * p.hq + head + r;
            mv[u] = p.ws_ml[2 * slot];
            lv[u] = p.ws_ml[2 * slot + 1];
            av[u] = p.ws_acc[slot * D + d];
          }
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            if (c0 + u < cend) {
              float ca, cb;
              bool keep;
              merge_stats(Mx, Lx, mv[u], lv[u], ca, cb, keep);
              Ax = merge_elem(Ax, av[u], keep, ca, cb);
            }
          }
        }
        const RowFinal fin(Lx, p.v_descale);
        buf_store2(orr, (uint32_t)e * 2u, bf16_bits(fin.elem<!FP8>(Ax)));
        if (d == 0) buf_store4(lr, (uint32_t)r * 4u, f32_bits(finalize_lse(Mx, Lx)));
      }
      return;
    }
  }
  run_blocks(std::false_type{});
  if constexpr (SPLIT) {
    store_partial<D, NT>(p, acc, m, l, dt0, chunk, q_start, head, nrows, rs, qrow, h);
  } else {
    store_output<D, NT, !FP8>(p, A, M, L, dt0, q_start, head, nrows, rs, qrow, h);
  }
}

template <int D, bool FP8, int NW, int WPE, bool WIN>
hipError_t launch_win(const PrefillParams& p, bool split, bool paged, dim3 grid, dim3 block,
                      hipStream_t stream) {
  if (paged) {
    if (split) {
      hipLaunchKernelGGL((prefill_kernel<D, FP8, NW, WPE, true, true, WIN>), grid, block, 0, stream, p);
    } else {
      hipLaunchKernelGGL((prefill_kernel<D, FP8, NW, WPE, false, true, WIN>), grid, block, 0, stream, p);
    }
  } else if (split) {
    hipLaunchKernelGGL((prefill_kernel<D, FP8, NW, WPE, true, false, WIN>), grid, block, 0, stream, p);
  } else {
    hipLaunchKernelGGL((prefill_kernel<D, FP8, NW, WPE, false, false, WIN>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

template <int D, bool FP8, int NW, int WPE>
hipError_t launch_one(const PrefillParams& p, bool split, bool paged, hipStream_t stream) {
  const long long per = (long long)p.batch * p.hq * p.tiles * (split ? p.cmax : 1);
  if (per <= 0) return hipSuccess;
  dim3 grid((unsigned)per), block(NW * kWave);
  if (p.window_left >= 0 || p.window_right >= 0)
    return launch_win<D, FP8, NW, WPE, true>(p, split, paged, grid, block, stream);
  return launch_win<D, FP8, NW, WPE, false>(p, split, paged, grid, block, stream);
}

// Per (head_dim, dtype): waves per workgroup and the waves per SIMD the
// register budget targets.  Eight waves (two per SIMD, so one wave's MFMAs can
// fill the other's gaps) up to D = 128, where a wave fits in the 256 registers
// that leaves it, and for fp8 D = 192, whose waves split the output columns
// (its scores are cheap on the 64-wide fp8 MFMA, so computing them twice costs
// less than a SIMD without a second wave); four waves (one per SIMD) for bf16
// D = 192.
template <int D, bool FP8>
struct Layout {
  static constexpr int kWaves = (D <= 128 || FP8) ? 8 : 4;
  static constexpr int kWavesPerEU = (D <= 128 || FP8) ? 2 : 1;
};

template <int D, bool FP8>
constexpr int tile_rows() {
  return PrefillCfg<D, FP8, Layout<D, FP8>::kWaves>::kTileRows;
}

template <int D, bool FP8>
hipError_t launch_layout(const PrefillParams& p, bool split, bool paged, hipStream_t stream) {
  using L = Layout<D, FP8>;
  return launch_one<D, FP8, L::kWaves, L::kWavesPerEU>(p, split, paged, stream);
}

}  // namespace

bool paged_extend_spreads(int head_dim, bool fp8) { return fp8 || head_dim <= 128; }

int prefill_tile_rows(int head_dim, bool fp8) {
  switch (head_dim) {
    case 64: return fp8 ? tile_rows<64, true>() : tile_rows<64, false>();
    case 128: return fp8 ? tile_rows<128, true>() : tile_rows<128, false>();
    case 192: return fp8 ? tile_rows<192, true>() : tile_rows<192, false>();
    default: return 32 * 8;
  }
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, bool fp8, bool split, bool paged,
                          hipStream_t stream) {
  switch (head_dim) {
    case 64:
      return fp8 ? launch_layout<64, true>(p, split, paged, stream)
                 : launch_layout<64, false>(p, split, paged, stream);
    case 128:
      return fp8 ? launch_layout<128, true>(p, split, paged, stream)
                 : launch_layout<128, false>(p, split, paged, stream);
    case 192:
      return fp8 ? launch_layout<192, true>(p, split, paged, stream)
                 : launch_layout<192, false>(p, split, paged, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace detattn
