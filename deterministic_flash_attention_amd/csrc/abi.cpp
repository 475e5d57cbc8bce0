// C-ABI entry points: host-side argument validation, then one launch per call.
// Every check runs before any HIP call, so a rejected call launches nothing and
// writes nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "../../include/detattn.h"
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

size_t partials_bytes_or_max(int64_t rows, int64_t hq, int64_t chunks, int64_t d) {
  if (rows < 0 || hq < 0 || chunks < 0 || d < 0) return 0;
  const long double n = (long double)rows * hq * chunks * (d + 2) * 4.0L;
  if (n > (long double)std::numeric_limits<size_t>::max() / 2) return std::numeric_limits<size_t>::max();
  return (size_t)rows * (size_t)hq * (size_t)chunks * (size_t)(d + 2) * 4u;
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

  const int tile = detattn::prefill_tile_rows(head_dim, dtype == DA_FP8_E4M3);
  if (((int64_t)max_seqlen_q + tile) * num_heads_q * head_dim * 4 > kMaxOffset) return DA_EUNSUPPORTED;
  const int32_t tiles = (int32_t)((max_seqlen_q + tile - 1) / tile);
  const int32_t cmax = chunks_for(max_context_len);
  if ((int64_t)batch * num_heads_q * tiles * (split ? cmax : 1) > kMaxOffset) return DA_EUNSUPPORTED;
  if (split && partials_bytes < partials_bytes_or_max(total_q, num_heads_q, cmax, head_dim))
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
  const hipError_t e = detattn::launch_prefill(p, head_dim, dtype == DA_FP8_E4M3, split, true,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ELAUNCH;
}

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
  if (dtype != DA_BF16 && dtype != DA_FP8_E4M3) return DA_EINVAL;
  if (schedule != DA_MONOLITHIC && schedule != DA_SPLIT) return DA_EINVAL;
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
  const bool split = schedule == DA_SPLIT;
  const int es = dtype == DA_FP8_E4M3 ? 1 : 2;
  if (!q || !k_cache || !v_cache || !page_table || !context_lens) return DA_EINVAL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(page_table, 4) || !aligned(context_lens, 4))
    return DA_EINVAL;
  if ((page_stride * es) % 16 || (token_stride * es) % 16 || (head_stride * es) % 16) return DA_EINVAL;
  if (!split && (!o || !aligned(o, 16) || (lse && !aligned(lse, 4)))) return DA_EINVAL;
  if (split && (!partials || !aligned(partials, 16))) return DA_EINVAL;
  const int32_t cmax = chunks_for(max_context_len);
  if ((int64_t)batch * num_heads_kv * (split ? cmax : 1) > kMaxOffset) return DA_EUNSUPPORTED;
  if (split && partials_bytes < partials_bytes_or_max(batch, num_heads_q, cmax, head_dim))
    return DA_EWORKSPACE;
  if (batch == 0 || (split && cmax == 0)) return DA_OK;

  detattn::DecodeParams p{};
  p.q = q;
  p.kc = k_cache;
  p.vc = v_cache;
  p.page_table = page_table;
  p.ctx_lens = context_lens;
  p.o = o;
  p.lse = lse;
  p.part_acc = partials;
  p.part_ml = partials ? partials + (size_t)cmax * batch * num_heads_q * head_dim : nullptr;
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

}  // extern "C"
