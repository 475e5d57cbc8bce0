// Internal launch interface between the C-ABI layer (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace detattn {

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  void* o;            // bf16 [total_q, hq, D]             (monolithic)
  float* lse;         // fp32 [total_q, hq] or null         (monolithic)
  float* part_acc;    // fp32 [cmax, total_q, hq, D]        (split)
  float* part_ml;     // fp32 [cmax, total_q, hq, 2]        (split)
  int64_t total_q;
  int64_t total_k;
  int32_t batch;
  int32_t hq;
  int32_t hkv;
  int32_t tiles;      // ceil(max_seqlen_q / tile rows)
  int32_t cmax;       // ceil(max_seqlen_k / 512)
  int32_t causal;
  int32_t window_left;   // sliding window on the bottom-right diagonal; -1 unbounded
  int32_t window_right;
  float c_scale;      // softmax_scale * q_descale * k_descale * log2(e)
  float v_descale;
  // Paged K/V (paged extend): k and v are the page caches, keys of sequence b
  // are its first ctx_lens[b] tokens, token j on page page_table[b][j / 16].
  const int32_t* page_table;  // [batch, max_pages]
  const int32_t* ctx_lens;    // [batch]
  int64_t num_pages;
  int64_t page_stride;        // elements
  int64_t token_stride;
  int64_t head_stride;
  int32_t max_pages;
  // Monolithic paged extend with a workspace: single-token sequences spread
  // their chunks over workgroups (null: no workspace).
  float* ws_acc;      // fp32 [cmax, batch, hq, D]
  float* ws_ml;       // fp32 [cmax, batch, hq, 2]
  int32_t* ws_cnt;    // int32 [batch, hkv], zero between launches
};

struct DecodeParams {
  const void* q;          // [batch, hq, D]
  const void* kc;         // paged caches, element strides below
  const void* vc;
  const int32_t* page_table;  // [batch, max_pages]
  const int32_t* ctx_lens;    // [batch]
  void* o;                // bf16 [batch, hq, D]              (monolithic)
  float* lse;             // fp32 [batch, hq] or null          (monolithic)
  float* part_acc;        // fp32 [cmax, batch, hq, D]         (split)
  float* part_ml;         // fp32 [cmax, batch, hq, 2]         (split)
  int64_t num_pages;
  int64_t page_stride;
  int64_t token_stride;
  int64_t head_stride;
  int32_t batch;
  int32_t hq;
  int32_t hkv;
  int32_t group;          // hq / hkv
  int32_t max_pages;
  int32_t cmax;           // ceil(max_context_len / 512)
  int32_t window_left;    // keys j >= ctx - 1 - window_left; -1 unbounded
  float c_scale;
  float v_descale;
};

struct MergeParams {
  const float* part_acc;  // fp32 [cmax, rows, hq, D]
  const float* part_ml;   // fp32 [cmax, rows, hq, 2]
  void* o;                // bf16 [rows, hq, D]
  float* lse;             // fp32 [rows, hq] or null
  int64_t rows;
  int32_t hq;
  int32_t cmax;
  float v_descale;
};

struct GemmParams {
  const void* a;          // bf16 [m, lda]
  const void* b;          // bf16 weight: [n, ldb] ([N, K] layout) or [k, ldb] ([K, N])
  void* c;                // bf16 [m, ldc]
  float* part;            // fp32 [nchunks, m, n]                 (split)
  int64_t lda, ldb, ldc;  // row strides in elements
  int64_t m, n, k;
  int32_t nchunks;        // ceil(k / 1024)
  int32_t tiles_m, tiles_n, group_m;  // set by the launcher (group_m: requested group)
};

// Each returns hipSuccess or the launch error.
hipError_t launch_prefill(const PrefillParams& p, int head_dim, bool fp8, bool split, bool paged,
                          hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int head_dim, bool fp8, bool split,
                         hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, int head_dim, hipStream_t stream);

// Whether the monolithic paged extend kernel of this configuration spreads
// single-token sequences over workgroups when given a workspace.
bool paged_extend_spreads(int head_dim, bool fp8);
int prefill_tile_rows(int head_dim, bool fp8);

// GEMM: config selects the tile shape (0 .. gemm_num_configs() - 1); every
// config computes the same bits.
hipError_t launch_gemm(const GemmParams& p, int config, bool kn, bool split, hipStream_t stream);
int gemm_num_configs();
void gemm_config_tile(int config, int* bm, int* bn);

}  // namespace detattn
