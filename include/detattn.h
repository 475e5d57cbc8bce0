/*
 * detattn — batch-invariant chunked flash-attention forward for MI355X (gfx950).
 *
 * The operation (RL-Kernel PR "MFMA batch-invariant GEMM and chunked Triton
 * attention", section 2 "Chunked-KV Triton flash attention") is
 *
 *     O = softmax(scale * Q K^T + mask) V
 *
 * served by one arithmetic path for full-sequence forward, prefill,
 * prefix-cached extend and single-token paged decode: keys are consumed in
 * 64-key blocks inside 512-key chunks, each chunk's online softmax starts from
 * an empty state, chunk partials are merged in ascending order with the exact
 * max/sum rescale, fully masked blocks leave a row untouched, and no
 * multiply-add is fused.  A monolithic schedule (one workgroup per query tile)
 * and a split schedule (one workgroup per sequence / head / chunk, then
 * attn_chunk_merge) give bit-identical rows, so a decode row equals the last row
 * of the prefill of the same sequence, and a row does not depend on which other
 * sequences share the batch.
 *
 * Conventions shared by every entry point
 *   - All tensors are caller-owned device memory, row-major and contiguous
 *     unless strides are given.  The library allocates nothing, keeps no state,
 *     never synchronises the host and launches only on `stream` (a hipStream_t;
 *     NULL is the null stream).  Calls on different streams may run concurrently.
 *   - Mask: key j of a sequence with L_q queries and L_k keys is visible from
 *     query row i iff j < L_k and (causal == 0 or j <= i + L_k - L_q), i.e.
 *     causal masks are aligned to the bottom-right corner.  A sliding window
 *     (local attention; window-sized bounds of the aiter MQA-logits page)
 *     window_left >= 0 further requires j >= i + L_k - L_q - window_left and
 *     window_right >= 0 requires j <= i + L_k - L_q + window_right, on the same
 *     diagonal; -1 leaves that side unbounded.  Keys outside a tile's window
 *     are never read.  A row with no visible key gets O = 0 and lse = -inf.
 *   - Grouped-query attention: query head h reads kv head h / (Hq / Hkv).
 *   - dtype DA_BF16: Q, K, V are bf16, all descales must be 1.0f.
 *     dtype DA_FP8_E4M3: Q, K, V are OCP E4M3FN codes with per-tensor fp32
 *     dequantisation scales (value = code * descale); scores use
 *     scale * q_descale * k_descale, P V runs in bf16 on exactly widened V, and
 *     the output is multiplied by v_descale.  O is always bf16.
 *   - lse (optional, may be NULL) is fp32, the natural log of
 *     sum_j exp(scale * q.k_j) over visible keys.
 *   - Stores never leave the valid cells: padded rows of a tile, rows of other
 *     sequences and cells outside [0, D) are not written, so whatever the caller
 *     pre-filled elsewhere in O survives.
 *   - Errors: arguments are checked on the host before anything is launched; a
 *     failing check returns its status with nothing launched and nothing
 *     written.  DA_ELAUNCH reports a launch failure.  Device-side values
 *     (cu_seqlens, context_lens, page tables) are not checked on the host; the
 *     kernels clamp every access to the extents passed here, so malformed
 *     values cannot read or write outside the given tensors.
 */
#ifndef DETATTN_H
#define DETATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DA_OK = 0,
  DA_EINVAL = 1,       /* malformed argument (null pointer, bad count, misalignment) */
  DA_EUNSUPPORTED = 2, /* well-formed but outside what the kernels implement */
  DA_EWORKSPACE = 3,   /* partials buffer too small */
  DA_ELAUNCH = 4       /* the HIP runtime rejected a launch */
} da_status;

typedef enum { DA_BF16 = 0, DA_FP8_E4M3 = 1 } da_dtype;
typedef enum { DA_MONOLITHIC = 0, DA_SPLIT = 1 } da_schedule;

#define DA_BLOCK_KEYS 64  /* keys per online-softmax update */
#define DA_CHUNK_KEYS 512 /* keys per chunk partial */
#define DA_PAGE_SIZE 16   /* tokens per KV-cache page */

/* Human-readable name of a status code (static storage, never NULL). */
const char* attn_status_str(int status);

/* Number of 512-key chunks for a key length: ceil(max_seqlen_k / 512), 0 for <= 0. */
int32_t attn_num_chunks(int32_t max_seqlen_k);

/* Bytes of the fp32 chunk-partial workspace for `rows` query rows:
 *   acc [max_chunks][rows][num_heads_q][head_dim] followed by
 *   ml  [max_chunks][rows][num_heads_q][2]   (m in log2 units, l).
 * Returns 0 for negative arguments and SIZE_MAX on overflow. */
size_t attn_partials_bytes(int64_t rows, int32_t num_heads_q, int32_t max_chunks,
                           int32_t head_dim);

/* Completion counters at the start of the monolithic paged extend's
 * workspace: DA_WORKSPACE_COUNTERS int32 words, 256 KiB, which must be zero
 * before the first call; every call leaves them zero, so one zero-filled
 * workspace can serve calls of any shape. */
#define DA_WORKSPACE_COUNTERS 65536

/* Bytes of the workspace that lets a monolithic attn_paged_extend_fwd spread
 * single-token sequences over workgroups: the counter region (one counter per
 * sequence and kv head, batch * num_heads_kv <= DA_WORKSPACE_COUNTERS), then
 * fp32 chunk partials
 *   acc [max_chunks][batch][num_heads_q][head_dim], then
 *   ml  [max_chunks][batch][num_heads_q][2].
 * Returns 0 for negative arguments and SIZE_MAX on overflow. */
size_t attn_extend_workspace_bytes(int32_t batch, int32_t num_heads_q, int32_t num_heads_kv,
                                   int32_t max_chunks, int32_t head_dim);

/*
 * Prefill / full-sequence forward / extend over packed variable-length
 * sequences (RL-Kernel page, section 2: one chunked arithmetic path for
 * full-sequence forward and prefill; head_dim 192 with E4M3FN inputs is the
 * ffpa-attn page's fp8 D=192 case, "Root cause" and "Verification").
 *   q        [total_q, Hq, D]   bf16 or E4M3FN codes
 *   k, v     [total_k, Hkv, D]  bf16 or E4M3FN codes
 *   cu_seqlens_q, cu_seqlens_k  device int32 [batch + 1] exclusive prefix sums;
 *            sequence b owns rows [cu_q[b], cu_q[b+1]) and keys [cu_k[b], cu_k[b+1]).
 *   max_seqlen_q, max_seqlen_k  host upper bounds of the per-sequence lengths.
 *   total_q, total_k            rows of q/o and of k/v; every access is clamped to them.
 *   head_dim  64, 128 or 192.
 *   schedule  DA_MONOLITHIC: writes o [total_q, Hq, D] bf16 and lse [total_q, Hq]
 *                            (lse may be NULL); partials are ignored.
 *             DA_SPLIT: writes the chunk partials of every row into `partials`
 *                       (layout of attn_partials_bytes with rows = total_q and
 *                       max_chunks = attn_num_chunks(max_seqlen_k)); o and lse are
 *                       not touched.  attn_chunk_merge then produces O.
 * Pointers q, k, v, o, partials must be 16-byte aligned; total_q must equal
 * cu_seqlens_q[batch] for the split schedule's merge to cover only written rows.
 */
da_status attn_prefill_fwd(int32_t dtype, const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                           int64_t total_q, int64_t total_k, int32_t num_heads_q,
                           int32_t num_heads_kv, int32_t head_dim, float softmax_scale,
                           int32_t causal, int32_t window_left, int32_t window_right,
                           float q_descale, float k_descale, float v_descale,
                           int32_t schedule, void* o, float* lse, float* partials,
                           size_t partials_bytes, void* stream);

/*
 * Single-token decode over a paged KV cache (RL-Kernel page, section 2:
 * single-token paged decode on the same arithmetic path, so a decode row
 * equals the last prefill row): sequence b's query (row b of q) is
 * the last token of a sequence of context_lens[b] tokens, so every cached key
 * j < context_lens[b] is visible (j >= context_lens[b] - 1 - window_left as well
 * when window_left >= 0; pages wholly below that are not read).  Token j of sequence b lives in page
 * page_table[b * max_pages_per_seq + j / 16] at slot j % 16.
 *   q         [batch, Hq, D]
 *   k_cache, v_cache  element (page, slot, kv_head, d) at
 *             page * page_stride + slot * token_stride + kv_head * head_stride + d
 *             (element strides; e.g. [num_pages, 16, Hkv, D] has 16*Hkv*D, Hkv*D, D).
 *   num_pages pages in each cache; table entries outside [0, num_pages) read as zero keys.
 *   page_table device int32 [batch, max_pages_per_seq]; context_lens device int32 [batch],
 *             each clamped to [0, max_pages_per_seq * 16].
 *   max_context_len  host upper bound of context_lens (sizes the chunk grid).
 *   page_size must be 16; Hq / Hkv must be at most 32.
 *   schedule  DA_SPLIT: one workgroup per (sequence, kv head, chunk) writes the
 *             partials (rows = batch, max_chunks = attn_num_chunks(max_context_len));
 *             follow with attn_chunk_merge on the same stream.
 *             DA_MONOLITHIC: one workgroup per (sequence, kv head) writes o [batch, Hq, D]
 *             and lse directly; bit-identical to split + merge.
 * Caches, q, o and partials must be 16-byte aligned and the byte strides
 * multiples of 16.  Keys past a sequence's context are never read, so dead
 * slots may hold anything (NaN included).
 */
da_status attn_decode_split_fwd(int32_t dtype, const void* q, const void* k_cache,
                                const void* v_cache, int64_t num_pages, int64_t page_stride,
                                int64_t token_stride, int64_t head_stride,
                                const int32_t* page_table, int32_t max_pages_per_seq,
                                const int32_t* context_lens, int32_t max_context_len,
                                int32_t window_left, int32_t batch, int32_t page_size,
                                int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                float softmax_scale, float q_descale, float k_descale,
                                float v_descale, int32_t schedule, float* partials,
                                size_t partials_bytes, void* o, float* lse, void* stream);

/*
 * Prefix-cached extend over a paged KV cache, for a batch that mixes prefill,
 * extend and decode sequences in one launch (RL-Kernel page, section 2: the
 * same arithmetic path serves prefill, prefix-cached extend and paged decode).
 * Sequence b has L_k = context_lens[b] cached tokens (its prefix and its new
 * tokens, already written to the cache) and L_q = cu_seqlens_q[b+1] -
 * cu_seqlens_q[b] query rows, which are its last L_q tokens: L_q = L_k is a
 * prefill, L_q < L_k an extend, L_q = 1 a decode step.  With causal == 1 row i
 * sees keys j <= i + L_k - L_q (bottom-right); with causal == 0 every cached key.
 *   q, cu_seqlens_q, total_q, max_seqlen_q  as for attn_prefill_fwd.
 *   k_cache, v_cache, num_pages, the strides, page_table, max_pages_per_seq,
 *   context_lens, max_context_len, page_size  as for attn_decode_split_fwd
 *            (no limit on Hq / Hkv here).
 *   schedule  as for attn_prefill_fwd, with max_chunks = attn_num_chunks(max_context_len).
 *   partials  DA_SPLIT: the chunk partials, as for attn_prefill_fwd.
 *             DA_MONOLITHIC: NULL, or a workspace of at least
 *             attn_extend_workspace_bytes(batch, Hq, Hkv, max_chunks, head_dim)
 *             bytes (DA_EWORKSPACE if smaller; DA_EUNSUPPORTED if
 *             batch * Hkv > DA_WORKSPACE_COUNTERS), 16-byte aligned.  With it, a
 *             single-token sequence whose context spans several chunks has its
 *             chunks dealt out to workgroups of the same launch that would
 *             otherwise be idle (the other query heads of its group times the
 *             launch's tile slots); each stores its chunks' partials there, and
 *             the last to finish (a device-scope counter per sequence and kv
 *             head) folds them and writes the rows.  Still one launch, and the
 *             same bits as without the workspace.  Its counter region must be
 *             zero before the first call (e.g. the buffer zero-filled once);
 *             every call leaves it zero.  Two calls in flight at once must not
 *             share a workspace.
 * Each row is bitwise equal to the same row computed by attn_prefill_fwd over
 * the gathered keys, and a decode row to attn_decode_split_fwd's, whichever
 * sequences share the launch.
 */
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
                                float* partials, size_t partials_bytes, void* stream);

/*
 * Fold chunk partials into O (RL-Kernel page, section 2: chunk partials merged
 * in ascending order with the exact FlashAttention-2 max/sum rescale, one bf16
 * rounding at the end): for every (row, head), partials c = 0 .. max_chunks-1
 * are merged left to right with the exact max/sum rescale (empty partials,
 * m = -inf, are skipped), then O = A / L (0 when L = 0) times v_descale is
 * rounded once to bf16.  o [rows, Hq, D] bf16, lse [rows, Hq] fp32 or NULL.
 * v_descale is 1.0f for bf16 inputs and the V scale for E4M3FN inputs.
 */
da_status attn_chunk_merge(const float* partials, size_t partials_bytes, int64_t rows,
                           int32_t num_heads_q, int32_t max_chunks, int32_t head_dim,
                           float v_descale, void* o, float* lse, void* stream);

/*
 * Allocation-free paged decode, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the split schedule of attn_decode_split_fwd followed by
 * attn_chunk_merge in one call, with the chunk partials kept in a static
 * device array of the library (DA_DECODE_SCRATCH_BYTES per GPU, held by every
 * GPU the library runs on until the process ends) instead of a caller
 * workspace.  Arguments are those of attn_decode_split_fwd without schedule
 * and partials; o [batch, Hq, D] bf16 and lse [batch, Hq] fp32 (may be NULL)
 * are caller-owned.  The result is bit-identical to split + merge (and to the
 * monolithic schedule).
 *   - Size limit: attn_partials_bytes(batch, Hq, attn_num_chunks(max_context_len),
 *     head_dim) must not exceed DA_DECODE_SCRATCH_BYTES, else DA_EWORKSPACE
 *     (checked on the host, nothing launched).
 *   - Calls no allocating routine (no hipMalloc, hipFree or memset).  The
 *     first call with a device current looks up that device's scratch
 *     address (hipGetSymbolAddress) and keeps it; `stream` must belong to the
 *     current device (DA_EINVAL otherwise).
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap on
 *     one GPU (different streams, or host threads without ordering) race and
 *     must be serialised by the caller.  Each call writes every partial it
 *     reads, so nothing left by an earlier call is ever read.
 */
#define DA_DECODE_SCRATCH_BYTES ((size_t)128 << 20)
da_status attn_decode_fwd_noalloc(int32_t dtype, const void* q, const void* k_cache,
                                  const void* v_cache, int64_t num_pages, int64_t page_stride,
                                  int64_t token_stride, int64_t head_stride,
                                  const int32_t* page_table, int32_t max_pages_per_seq,
                                  const int32_t* context_lens, int32_t max_context_len,
                                  int32_t window_left, int32_t batch, int32_t page_size,
                                  int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                  float softmax_scale, float q_descale, float k_descale,
                                  float v_descale, void* o, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DETATTN_H */
