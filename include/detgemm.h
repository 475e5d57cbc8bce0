/*
 * detgemm — batch-invariant bf16 GEMM for MI355X (gfx950), in libdetattn.so.
 *
 * The operation (RL-Kernel PR "MFMA batch-invariant GEMM and chunked Triton
 * attention", section 1 "MFMA batch-invariant deterministic GEMM") is
 *
 *     C[M, N] = A[M, K] W^T      (weight W stored [N, K], the layer-weight view)
 *     C[M, N] = A[M, K] W        (weight W stored [K, N], the prepared layout)
 *
 * with bf16 operands, fp32 accumulation and one rounding of the result to bf16
 * (round to nearest even).  The summation order is fixed and is the contract:
 *   - every product runs on one pinned MFMA shape, v_mfma_f32_32x32x16_bf16;
 *     MFMA step s of K block b covers K indices 64 b + 16 s + [0, 16);
 *   - K is consumed in ascending 64-wide blocks inside fixed 1024-wide chunks;
 *     each chunk's partial starts from +0;
 *   - chunk partials are combined left to right in fp32 (total = p_0, then
 *     total = total + p_c), then rounded once.
 * Each output element therefore depends only on its row of A and its column of
 * W: the tile shape (`config`), M, the row strides, the weight layout and the
 * schedule (monolithic, or split over chunks followed by a combine pass) all
 * give bit-identical results.  K past the last multiple of 64 is padded with
 * zeros inside the last block.
 *
 * Conventions
 *   - All tensors are caller-owned device memory, row-major with the given row
 *     strides (in elements).  The library allocates nothing, keeps no state,
 *     never synchronises the host and launches only on `stream` (a hipStream_t;
 *     NULL is the null stream).
 *   - Requirements: N and K multiples of 8; lda, ldw, ldc multiples of 8 with
 *     lda >= K, ldc >= N, ldw >= K ([N, K]) or ldw >= N ([K, N]); A, W, C and
 *     the workspace 16-byte aligned.  M is arbitrary.  Only C[0:M, 0:N] is
 *     written.
 *   - K = 0 gives C = +0.  M = 0 or N = 0 launches nothing.
 *   - Errors use the da_status codes of detattn.h: every check runs on the host
 *     before anything is launched, so a failing call writes nothing.
 *     DA_EUNSUPPORTED: N or K not a multiple of 8, or a tile's byte extent
 *     beyond 2^31 (row strides above about four million elements).
 */
#ifndef DETGEMM_H
#define DETGEMM_H

#include <stddef.h>
#include <stdint.h>

#include "detattn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DG_WEIGHT_NK = 0, DG_WEIGHT_KN = 1 } dg_weight_layout;

#define DG_BLOCK_K 64   /* K per MFMA chain block */
#define DG_CHUNK_K 1024 /* K per chunk partial */

/* ceil(k / 1024): the number of chunk partials; 0 for k <= 0. */
int32_t det_gemm_num_chunks(int64_t k);

/* Bytes of fp32 workspace the split schedule needs: num_chunks(k) * m * n * 4. */
size_t det_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* Number of tile configurations; config c in [0, n) has tile bm x bn.  All give
 * the same bits; they differ only in speed. */
int32_t det_gemm_num_configs(void);
da_status det_gemm_config_tile(int32_t config, int32_t* bm, int32_t* bn);

/* C = A W^T (weight_layout DG_WEIGHT_NK, W is [N, ldw]) or C = A W
 * (DG_WEIGHT_KN, W is [K, ldw]); A is [M, lda], C is [M, ldc], all bf16.
 *
 * schedule DA_MONOLITHIC: one workgroup per output tile runs every chunk and
 *   the left fold in registers; `workspace` may be NULL.
 * schedule DA_SPLIT: one workgroup per (tile, chunk) stores the fp32 chunk
 *   partial into `workspace` ([num_chunks, M, N], at least
 *   det_gemm_workspace_bytes(m, n, k) bytes), then a combine pass folds the
 *   partials in ascending order and rounds.  Meant for small M (decode), where
 *   the tiles alone do not fill the GPU.
 * config: a tile configuration index, or -1 to let the library choose.
 */
da_status det_gemm_fwd(const void* a, int64_t lda, const void* w, int64_t ldw,
                       int32_t weight_layout, void* c, int64_t ldc, int64_t m, int64_t n,
                       int64_t k, int32_t schedule, int32_t config, float* workspace,
                       size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DETGEMM_H */
