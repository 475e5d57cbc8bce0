// C-ABI entry points: host-side argument validation, then one launch per call.
// Every check runs before any HIP call, so a rejected call launches nothing and
// writes nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>
#include <mutex>

#include "../../include/detattn.h"
#include "../../include/detgemm.h"
#include "kernels.hpp"

namespace {

constexpr int64_t kMaxOffset = 0x7FFFFFFF;  // byte offsets inside one descriptor
constexpr double kLog2e = 1.4426950408889634;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }
bool supported_dim(int32_t d) { return d == 64 || d == 128 || d == 192; }
int32_t chunks_for(int64_t keys) { return keys <= 0 ? 0 : (int32_t)((keys + 511) / 512); }

// The single fp32 score constant every kernel multiplies by; computed the same
// way for every entry point so all schedules see identical bits.
float score_constant(float scale, float qd, float kd) {
  return (float)((double)scale * (double)qd * (double)kd * kLog2e);
}

bool check_descales(int32_t dtype, float qd, float kd, float vd) {
  if (dtype == DA_BF16) return qd == 1.0f && kd == 1.0f && vd == 1.0f;
  return finite_pos(qd) && finite_pos(kd) && finite_pos(vd);
}

// Completion counters at the start of a workspace: a fixed region, so that
// calls of any shape find theirs where every earlier call left zeros.
constexpr size_t kCounterBytes = (size_t)DA_WORKSPACE_COUNTERS * 4u;

size_t partials_bytes_or_max(int64_t rows, int64_t hq, int64_t chunks, int64_t d) {
  if (rows < 0 || hq < 0 || chunks < 0 || d < 0) return 0;
  const long double n = (long double)rows * hq * chunks * (d + 2) * 4.0L;
  if (n > (long double)std::numeric_limits<size_t>::max() / 2) return std::numeric_limits<size_t>::max();
  return (size_t)rows * (size_t)hq * (size_t)chunks * (size_t)(d + 2) * 4u;
}

int32_t gemm_chunks(int64_t k) { return k <= 0 ? 0 : (int32_t)((k + DG_CHUNK_K - 1) / DG_CHUNK_K); }

// Tile shape when the caller leaves it open.  Every choice computes the same
// bits.  The large tiles want two waves per SIMD and 512 launches or more:
// when N has no ragged 192-column tail, 256 x 192 (eight waves, one workgroup
// per CU) or else 128 x 192 (four waves, two per CU); otherwise 128 x 128.
// Smaller problems take the largest tile whose launch (tiles x split factor)
// still covers the 256 compute units, else the one with the most workgroups.
int64_t gemm_launch_count(int32_t cfg, int64_t m, int64_t n, int64_t split_factor) {
  int bm = 0, bn = 0;
  detattn::gemm_config_tile(cfg, &bm, &bn);
  return ((m + bm - 1) / bm) * ((n + bn - 1) / bn) * split_factor;
}

int32_t gemm_auto_config(int64_t m, int64_t n, int64_t split_factor) {
  if (n % 192 == 0 && gemm_launch_count(5, m, n, split_factor) >= 512) return 5;
  if (n % 192 == 0 && gemm_launch_count(0, m, n, split_factor) >= 512) return 0;
  if (gemm_launch_count(1, m, n, split_factor) >= 512) return 1;
  int32_t best = 1;
  int64_t best_count = -1;
  for (int32_t cfg = 1; cfg <= 4; ++cfg) {
    const int64_t count = gemm_launch_count(cfg, m, n, split_factor);
    if (count >= 256) return cfg;
    if (count > best_count) {
      best = cfg;
      best_count = count;
    }
  }
  return best;
}

// Device scratch of the allocation-free decode entry point: the split
// schedule's chunk partials of one call live here instead of in a caller
// workspace.  Every GPU the library runs on holds its own copy for the life
// of the process.  In host code `scratch` is only a host-side stand-in: its
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and only that address is passed to kernels.
constexpr size_t kScratchBytes = DA_DECODE_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device (looked up on the first call
// made with that device current).
hipError_t scratch_on_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* attn_status_str(int status) {
  switch (status) {
    case DA_OK: return "DA_OK";
    case DA_EINVAL: return "DA_EINVAL: malformed argument";
    case DA_EUNSUPPORTED: return "DA_EUNSUPPORTED: configuration not implemented";
    case DA_EWORKSPACE: return "DA_EWORKSPACE: partials buffer too small";
    case DA_ELAUNCH: return "DA_ELAUNCH: kernel launch failed";
    default: return "unknown status";
  }
}

int32_t attn_num_chunks(int32_t max_seqlen_k) { return chunks_for(max_seqlen_k); }

size_t attn_partials_bytes(int64_t rows, int32_t num_heads_q, int32_t max_chunks,
                           int32_t head_dim) {
  return partials_bytes_or_max(rows, num_heads_q, max_chunks, head_dim);
}

size_t attn_extend_workspace_bytes(int32_t batch, int32_t num_heads_q, int32_t num_heads_kv,
                                   int32_t max_chunks, int32_t head_dim) {
  if (batch < 0 || num_heads_kv < 0 || num_heads_q < 0 || max_chunks < 0 || head_dim < 0) return 0;
  const size_t cells = partials_bytes_or_max(batch, num_heads_q, max_chunks, head_dim);
  if (cells == std::numeric_limits<size_t>::max()) return cells;
  // The counter region (one int32 per sequence and kv head) first, at a fixed
  // size, then the partials.
  return kCounterBytes + cells;
}

da_status attn_prefill_fwd(int32_t dtype, const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                           int64_t total_q, int64_t total_k, int32_t num_heads_q,
                           int32_t num_heads_kv, int32_t head_dim, float softmax_scale,
                           int32_t causal, int32_t window_left, int32_t window_right,
                           float q_descale, float k_descale, float v_descale,
                           int32_t schedule, void* o, float* lse, float* partials,
                           size_t partials_bytes, void* stream) {
  if (dtype != DA_BF16 && dtype != DA_FP8_E4M3) return DA_EINVAL;
  if (schedule != DA_MONOLITHIC && schedule != DA_SPLIT) return DA_EINVAL;
  if (causal != 0 && causal != 1) return DA_EINVAL;
  if (window_left < -1 || window_right < -1) return DA_EINVAL;
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return DA_EINVAL;
  if (num_heads_q <= 0 || num_heads_kv <= 0 || num_heads_q % num_heads_kv != 0) return DA_EINVAL;
  if (!supported_dim(head_dim)) return DA_EUNSUPPORTED;
  if (!finite_pos(softmax_scale)) return DA_EINVAL;
  if (!check_descales(dtype, q_descale, k_descale, v_descale)) return DA_EINVAL;
  const bool split = schedule == DA_SPLIT;
  if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_k) return DA_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(cu_seqlens_q, 4) ||
      !aligned(cu_seqlens_k, 4))
    return DA_EINVAL;
  if (!split && (!o || !aligned(o, 16) || (lse && !aligned(lse, 4)))) return DA_EINVAL;
  if (split && (!partials || !aligned(partials, 16))) return DA_EINVAL;

  const int es = dtype == DA_FP8_E4M3 ? 1 : 2;
  const int tile = detattn::prefill_tile_rows(head_dim, dtype == DA_FP8_E4M3);
  // 32-bit descriptor offsets: rows of one sequence (plus a padded tile) for the
  // widest per-row record (fp32 partial accumulators), and the key rows.
  if (((int64_t)max_seqlen_q + tile) * num_heads_q * head_dim * 4 > kMaxOffset) return DA_EUNSUPPORTED;
  if (((int64_t)max_seqlen_k + 64) * num_heads_kv * head_dim * es > kMaxOffset) return DA_EUNSUPPORTED;
  const int32_t tiles = (int32_t)((max_seqlen_q + tile - 1) / tile);
  const int32_t cmax = chunks_for(max_seqlen_k);
  if ((int64_t)batch * num_heads_q * tiles * (split ? cmax : 1) > kMaxOffset) return DA_EUNSUPPORTED;
  if (split && partials_bytes < partials_bytes_or_max(total_q, num_heads_q, cmax, head_dim))
    return DA_EWORKSPACE;
  if (batch == 0 || tiles == 0 || (split && cmax == 0)) return DA_OK;

  detattn::PrefillParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.o = o;
  p.lse = lse;
  p.part_acc = partials;
  p.part_ml = partials ? partials + (size_t)cmax * total_q * num_heads_q * head_dim : nullptr;
  p.total_q = total_q;
  p.total_k = total_k;
  p.batch = batch;
  p.hq = num_heads_q;
  p.hkv = num_heads_kv;
  p.tiles = tiles;
  p.cmax = cmax;
  p.causal = causal;
  p.window_left = window_left;
  p.window_right = window_right;
  p.c_scale = score_constant(softmax_scale, q_descale, k_descale);
  p.v_descale = v_descale;
  const hipError_t e = detattn::launch_prefill(p, head_dim, dtype == DA_FP8_E4M3, split, false,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ELAUNCH;
}

da_status attn_paged_extend_fwd(int32_t dtype, const void* q, const int32_t* cu_seqlens_q,
                                const void* k_cache, const void* v_cache, int64_t num_pages,
                                int64_t page_stride, int64_t token_stride, int64_t head_stride,
                                const int32_t* page_table, int32_t max_pages_per_seq,
                                const int32_t* context_lens, int32_t batch, int32_t max_seqlen_q,
                                int32_t max_context_len, int64_t total_q, int32_t page_size,
                                int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                float softmax_scale, int32_t causal, int32_t window_left,
                                int32_t window_right, float q_descale, float k_descale,
                                float v_descale, int32_t schedule, void* o, float* lse,
                                float* partials, size_t partials_bytes, void* stream) {
  if (dtype != DA_BF16 && dtype != DA_FP8_E4M3) return DA_EINVAL;
  if (schedule != DA_MONOLITHIC && schedule != DA_SPLIT) return DA_EINVAL;
  if (causal != 0 && causal != 1) return DA_EINVAL;
  if (window_left < -1 || window_right < -1) return DA_EINVAL;
  if (batch < 0 || max_seqlen_q < 0 || max_context_len < 0 || total_q < 0) return DA_EINVAL;
  if (max_pages_per_seq <= 0 || num_pages <= 0) return DA_EINVAL;
  if (page_stride <= 0 || token_stride <= 0 || head_stride <= 0) return DA_EINVAL;
  if (num_heads_q <= 0 || num_heads_kv <= 0 || num_heads_q % num_heads_kv != 0) return DA_EINVAL;
  if (page_size != DA_PAGE_SIZE) return DA_EUNSUPPORTED;
  if (!supported_dim(head_dim)) return DA_EUNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_pages_per_seq * DA_PAGE_SIZE) return DA_EINVAL;
  if (!finite_pos(softmax_scale)) return DA_EINVAL;
  if (!check_descales(dtype, q_descale, k_descale, v_descale)) return DA_EINVAL;
  const bool split = schedule == DA_SPLIT;
  const int es = dtype == DA_FP8_E4M3 ? 1 : 2;
  if (!q || !cu_seqlens_q || !k_cache || !v_cache || !page_table || !context_lens) return DA_EINVAL;
  if (!aligned(q, 16) || !aligned(cu_seqlens_q, 4) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(page_table, 4) || !aligned(context_lens, 4))
    return DA_EINVAL;
  if ((page_stride * es) % 16 || (token_stride * es) % 16 || (head_stride * es) % 16) return DA_EINVAL;
  // A token's head row must not overlap the next token's; a page's tokens are
  // addressed with 32-bit offsets.
  if (token_stride < head_dim) return DA_EINVAL;
  if (token_stride * es * DA_PAGE_SIZE > kMaxOffset) return DA_EUNSUPPORTED;
  if (!split && (!o || !aligned(o, 16) || (lse && !aligned(lse, 4)))) return DA_EINVAL;
  if (split && (!partials || !aligned(partials, 16))) return DA_EINVAL;
  if (!split && partials && !aligned(partials, 16)) return DA_EINVAL;

  const int tile = detattn::prefill_tile_rows(head_dim, dtype == DA_FP8_E4M3);
  if (((int64_t)max_seqlen_q + tile) * num_heads_q * head_dim * 4 > kMaxOffset) return DA_EUNSUPPORTED;
  const int32_t cmax = chunks_for(max_context_len);
  int32_t tiles = (int32_t)((max_seqlen_q + tile - 1) / tile);
  if (!split && partials && max_seqlen_q > 0 &&
      detattn::paged_extend_spreads(head_dim, dtype == DA_FP8_E4M3)) {
    // Chunk spread: a single-token sequence's tile set (the query heads of a
    // kv group, packed in one tile, or one head without grouping) gets a
    // workgroup slot per chunk; the launch's tile slots grow to that.
    const int32_t group = num_heads_q / num_heads_kv;
    const int32_t tset = group > 1 ? group : 1;
    tiles = std::max(tiles, (cmax + tset - 1) / tset);  // enough for runs of any length
  }
  if ((int64_t)batch * num_heads_q * tiles * (split ? cmax : 1) > kMaxOffset) return DA_EUNSUPPORTED;
  if (split && partials_bytes < partials_bytes_or_max(total_q, num_heads_q, cmax, head_dim))
    return DA_EWORKSPACE;
  if (!split && partials && (int64_t)batch * num_heads_kv > DA_WORKSPACE_COUNTERS)
    return DA_EUNSUPPORTED;
  if (!split && partials &&
      partials_bytes < attn_extend_workspace_bytes(batch, num_heads_q, num_heads_kv, cmax, head_dim))
    return DA_EWORKSPACE;
  if (batch == 0 || tiles == 0 || (split && cmax == 0)) return DA_OK;

  detattn::PrefillParams p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.cu_q = cu_seqlens_q;
  p.cu_k = nullptr;
  p.o = o;
  p.lse = lse;
  p.part_acc = partials;
  p.part_ml = partials ? partials + (size_t)cmax * total_q * num_heads_q * head_dim : nullptr;
  p.total_q = total_q;
  p.total_k = 0;
  p.batch = batch;
  p.hq = num_heads_q;
  p.hkv = num_heads_kv;
  p.tiles = tiles;
  p.cmax = cmax;
  p.causal = causal;
  p.window_left = window_left;
  p.window_right = window_right;
  p.c_scale = score_constant(softmax_scale, q_descale, k_descale);
  p.v_descale = v_descale;
  p.page_table = page_table;
  p.ctx_lens = context_lens;
  p.num_pages = num_pages;
  p.page_stride = page_stride;
  p.token_stride = token_stride;
  p.head_stride = head_stride;
  p.max_pages = max_pages_per_seq;
  if (!split && partials) {
    // Monolithic with a workspace: chunk partials of spread single-token
    // sequences, then their counters.
    const size_t cells = (size_t)cmax * batch * num_heads_q;
    p.ws_cnt = reinterpret_cast<int32_t*>(partials);
    p.ws_acc = partials + kCounterBytes / 4;
    p.ws_ml = p.ws_acc + cells * head_dim;
    p.part_acc = nullptr;
    p.part_ml = nullptr;
  }
  const hipError_t e = detattn::launch_prefill(p, head_dim, dtype == DA_FP8_E4M3, split, true,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ELAUNCH;
}

}  // extern "C"

namespace {

// Validation and parameters shared by the paged decode entry points.  Runs no
// HIP call.  *cmax receives the chunk count of the split schedule.
da_status decode_setup(int32_t dtype, const void* q, const void* k_cache, const void* v_cache,
                       int64_t num_pages, int64_t page_stride, int64_t token_stride,
                       int64_t head_stride, const int32_t* page_table, int32_t max_pages_per_seq,
                       const int32_t* context_lens, int32_t max_context_len, int32_t window_left,
                       int32_t batch, int32_t page_size, int32_t num_heads_q,
                       int32_t num_heads_kv, int32_t head_dim, float softmax_scale,
                       float q_descale, float k_descale, float v_descale, bool split,
                       detattn::DecodeParams* out, int32_t* cmax_out) {
  if (dtype != DA_BF16 && dtype != DA_FP8_E4M3) return DA_EINVAL;
  if (window_left < -1) return DA_EINVAL;
  if (batch < 0 || max_context_len < 0 || max_pages_per_seq <= 0 || num_pages <= 0) return DA_EINVAL;
  if (page_stride <= 0 || token_stride <= 0 || head_stride <= 0) return DA_EINVAL;
  if (num_heads_q <= 0 || num_heads_kv <= 0 || num_heads_q % num_heads_kv != 0) return DA_EINVAL;
  if (page_size != DA_PAGE_SIZE) return DA_EUNSUPPORTED;
  if (!supported_dim(head_dim)) return DA_EUNSUPPORTED;
  if (num_heads_q / num_heads_kv > 32) return DA_EUNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_pages_per_seq * DA_PAGE_SIZE) return DA_EINVAL;
  if (!finite_pos(softmax_scale)) return DA_EINVAL;
  if (!check_descales(dtype, q_descale, k_descale, v_descale)) return DA_EINVAL;
  const int es = dtype == DA_FP8_E4M3 ? 1 : 2;
  if (!q || !k_cache || !v_cache || !page_table || !context_lens) return DA_EINVAL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(page_table, 4) || !aligned(context_lens, 4))
    return DA_EINVAL;
  if ((page_stride * es) % 16 || (token_stride * es) % 16 || (head_stride * es) % 16) return DA_EINVAL;
  const int32_t cmax = chunks_for(max_context_len);
  if ((int64_t)batch * num_heads_kv * (split ? cmax : 1) > kMaxOffset) return DA_EUNSUPPORTED;

  detattn::DecodeParams& p = *out;
  p = detattn::DecodeParams{};
  p.q = q;
  p.kc = k_cache;
  p.vc = v_cache;
  p.page_table = page_table;
  p.ctx_lens = context_lens;
  p.num_pages = num_pages;
  p.page_stride = page_stride;
  p.token_stride = token_stride;
  p.head_stride = head_stride;
  p.batch = batch;
  p.hq = num_heads_q;
  p.hkv = num_heads_kv;
  p.group = num_heads_q / num_heads_kv;
  p.max_pages = max_pages_per_seq;
  p.cmax = cmax;
  p.window_left = window_left;
  p.c_scale = score_constant(softmax_scale, q_descale, k_descale);
  p.v_descale = v_descale;
  *cmax_out = cmax;
  return DA_OK;
}

}  // namespace

extern "C" {

da_status attn_decode_split_fwd(int32_t dtype, const void* q, const void* k_cache,
                                const void* v_cache, int64_t num_pages, int64_t page_stride,
                                int64_t token_stride, int64_t head_stride,
                                const int32_t* page_table, int32_t max_pages_per_seq,
                                const int32_t* context_lens, int32_t max_context_len,
                                int32_t window_left, int32_t batch, int32_t page_size,
                                int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                float softmax_scale, float q_descale, float k_descale,
                                float v_descale, int32_t schedule, float* partials,
                                size_t partials_bytes, void* o, float* lse, void* stream) {
  if (schedule != DA_MONOLITHIC && schedule != DA_SPLIT) return DA_EINVAL;
  const bool split = schedule == DA_SPLIT;
  detattn::DecodeParams p{};
  int32_t cmax = 0;
  const da_status st = decode_setup(dtype, q, k_cache, v_cache, num_pages, page_stride,
                                    token_stride, head_stride, page_table, max_pages_per_seq,
                                    context_lens, max_context_len, window_left, batch, page_size,
                                    num_heads_q, num_heads_kv, head_dim, softmax_scale, q_descale,
                                    k_descale, v_descale, split, &p, &cmax);
  if (st != DA_OK) return st;
  if (!split && (!o || !aligned(o, 16) || (lse && !aligned(lse, 4)))) return DA_EINVAL;
  if (split && (!partials || !aligned(partials, 16))) return DA_EINVAL;
  if (split && partials_bytes < partials_bytes_or_max(batch, num_heads_q, cmax, head_dim))
    return DA_EWORKSPACE;
  if (batch == 0 || (split && cmax == 0)) return DA_OK;
  p.o = o;
  p.lse = lse;
  p.part_acc = partials;
  p.part_ml = partials ? partials + (size_t)cmax * batch * num_heads_q * head_dim : nullptr;
  const hipError_t e = detattn::launch_decode(p, head_dim, dtype == DA_FP8_E4M3, split,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ELAUNCH;
}

da_status attn_chunk_merge(const float* partials, size_t partials_bytes, int64_t rows,
                           int32_t num_heads_q, int32_t max_chunks, int32_t head_dim,
                           float v_descale, void* o, float* lse, void* stream) {
  if (rows < 0 || num_heads_q <= 0 || max_chunks < 0) return DA_EINVAL;
  if (!supported_dim(head_dim)) return DA_EUNSUPPORTED;
  if (!finite_pos(v_descale)) return DA_EINVAL;
  if (rows > 0 && (!o || !aligned(o, 16) || (lse && !aligned(lse, 4)))) return DA_EINVAL;
  if (rows > 0 && max_chunks > 0 && (!partials || !aligned(partials, 16))) return DA_EINVAL;
  if (partials_bytes < partials_bytes_or_max(rows, num_heads_q, max_chunks, head_dim))
    return DA_EWORKSPACE;
  if (rows * (int64_t)num_heads_q > (int64_t)kMaxOffset * 4) return DA_EUNSUPPORTED;
  if (rows == 0) return DA_OK;
  detattn::MergeParams p{};
  p.part_acc = partials;
  p.part_ml = partials ? partials + (size_t)max_chunks * rows * num_heads_q * head_dim : nullptr;
  p.o = o;
  p.lse = lse;
  p.rows = rows;
  p.hq = num_heads_q;
  p.cmax = max_chunks;
  p.v_descale = v_descale;
  const hipError_t e = detattn::launch_merge(p, head_dim, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ELAUNCH;
}

da_status attn_decode_fwd_noalloc(int32_t dtype, const void* q, const void* k_cache,
                                  const void* v_cache, int64_t num_pages, int64_t page_stride,
                                  int64_t token_stride, int64_t head_stride,
                                  const int32_t* page_table, int32_t max_pages_per_seq,
                                  const int32_t* context_lens, int32_t max_context_len,
                                  int32_t window_left, int32_t batch, int32_t page_size,
                                  int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                  float softmax_scale, float q_descale, float k_descale,
                                  float v_descale, void* o, float* lse, void* stream) {
  detattn::DecodeParams p{};
  int32_t cmax = 0;
  const da_status st = decode_setup(dtype, q, k_cache, v_cache, num_pages, page_stride,
                                    token_stride, head_stride, page_table, max_pages_per_seq,
                                    context_lens, max_context_len, window_left, batch, page_size,
                                    num_heads_q, num_heads_kv, head_dim, softmax_scale, q_descale,
                                    k_descale, v_descale, true, &p, &cmax);
  if (st != DA_OK) return st;
  if (!o || !aligned(o, 16) || (lse && !aligned(lse, 4))) return DA_EINVAL;
  if (partials_bytes_or_max(batch, num_heads_q, cmax, head_dim) > kScratchBytes)
    return DA_EWORKSPACE;
  if (batch == 0) return DA_OK;
  if (stream != nullptr) {
    // The scratch address belongs to the current device; so must the stream.
    int cur = -1;
    hipDevice_t sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess ||
        hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return DA_ELAUNCH;
    if (sdev != cur) return DA_EINVAL;
  }
  float* part = nullptr;
  if (scratch_on_current_device(&part) != hipSuccess) return DA_ELAUNCH;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (cmax > 0) {
    // Split: every chunk slot c < cmax of every (row, head) is written (empty
    // chunks as m = -inf, l = 0), so nothing left by an earlier call is read.
    p.part_acc = part;
    p.part_ml = part + (size_t)cmax * batch * num_heads_q * head_dim;
    hipError_t e = detattn::launch_decode(p, head_dim, dtype == DA_FP8_E4M3, true, hs);
    if (e != hipSuccess) return DA_ELAUNCH;
  }
  detattn::MergeParams mp{};
  mp.part_acc = part;
  mp.part_ml = part + (size_t)cmax * batch * num_heads_q * head_dim;
  mp.o = o;
  mp.lse = lse;
  mp.rows = batch;
  mp.hq = num_heads_q;
  mp.cmax = cmax;
  mp.v_descale = v_descale;
  const hipError_t e = detattn::launch_merge(mp, head_dim, hs);
  return e == hipSuccess ? DA_OK : DA_ELAUNCH;
}

// ---- batch-invariant GEMM ------------------------------------------------------

int32_t det_gemm_num_chunks(int64_t k) { return gemm_chunks(k); }

size_t det_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k < 0) return 0;
  const long double b = (long double)gemm_chunks(k) * m * n * 4.0L;
  if (b > (long double)std::numeric_limits<size_t>::max() / 2) return std::numeric_limits<size_t>::max();
  return (size_t)gemm_chunks(k) * (size_t)m * (size_t)n * 4u;
}

int32_t det_gemm_num_configs(void) { return detattn::gemm_num_configs(); }

da_status det_gemm_config_tile(int32_t config, int32_t* bm, int32_t* bn) {
  if (config < 0 || config >= detattn::gemm_num_configs() || !bm || !bn) return DA_EINVAL;
  int m = 0, n = 0;
  detattn::gemm_config_tile(config, &m, &n);
  *bm = m;
  *bn = n;
  return DA_OK;
}

da_status det_gemm_fwd(const void* a, int64_t lda, const void* w, int64_t ldw,
                       int32_t weight_layout, void* c, int64_t ldc, int64_t m, int64_t n,
                       int64_t k, int32_t schedule, int32_t config, float* workspace,
                       size_t workspace_bytes, void* stream) {
  if (weight_layout != DG_WEIGHT_NK && weight_layout != DG_WEIGHT_KN) return DA_EINVAL;
  if (schedule != DA_MONOLITHIC && schedule != DA_SPLIT) return DA_EINVAL;
  if (m < 0 || n < 0 || k < 0) return DA_EINVAL;
  if (config < -1 || config >= detattn::gemm_num_configs()) return DA_EINVAL;
  if (n % 8 || k % 8) return DA_EUNSUPPORTED;
  const bool kn = weight_layout == DG_WEIGHT_KN;
  const bool split = schedule == DA_SPLIT;
  if (m == 0 || n == 0) return DA_OK;
  if (!c || !aligned(c, 16) || ldc < n || ldc % 8) return DA_EINVAL;
  if (k > 0) {
    if (!a || !aligned(a, 16) || lda < k || lda % 8) return DA_EINVAL;
    if (!w || !aligned(w, 16) || ldw < (kn ? n : k) || ldw % 8) return DA_EINVAL;
  }
  const int32_t nchunks = gemm_chunks(k);
  if (split && nchunks > 0) {
    if (!workspace || !aligned(workspace, 16)) return DA_EINVAL;
    if (workspace_bytes < det_gemm_workspace_bytes(m, n, k)) return DA_EWORKSPACE;
  }
  if (config < 0) config = gemm_auto_config(m, n, split ? nchunks : 1);
  int32_t bm = 0, bn = 0;
  det_gemm_config_tile(config, &bm, &bn);
  // Every byte offset inside one tile's descriptor must stay below 2^31.
  const int64_t tiles = ((m + bm - 1) / bm) * ((n + bn - 1) / bn);
  // Grid sizes: the tile grid, and the combine pass's one workgroup per 1024
  // columns of a row.
  if (tiles > kMaxOffset || m * ((n + 1023) / 1024) > kMaxOffset) return DA_EUNSUPPORTED;
  if (k > 0) {
    if (((bm - 1) * lda + k) * 2 > kMaxOffset) return DA_EUNSUPPORTED;
    if (kn ? (k * ldw + bn) * 2 > kMaxOffset : ((bn - 1) * ldw + k) * 2 > kMaxOffset)
      return DA_EUNSUPPORTED;
  }
  if (((bm - 1) * ldc + bn) * 2 > kMaxOffset) return DA_EUNSUPPORTED;
  if (split && ((bm - 1) * n + bn) * 4 > kMaxOffset) return DA_EUNSUPPORTED;

  detattn::GemmParams p{};
  p.a = a;
  p.b = w;
  p.c = c;
  p.part = workspace;
  p.lda = lda;
  p.ldb = ldw;
  p.ldc = ldc;
  p.m = m;
  p.n = n;
  p.k = k;
  p.nchunks = nchunks;
  p.group_m = 8;
  const hipError_t e =
      detattn::launch_gemm(p, config, kn, split, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ELAUNCH;
}

}  // extern "C"
