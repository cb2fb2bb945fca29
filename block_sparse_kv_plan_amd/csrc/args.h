// Launch-argument structs and constants shared by host dispatch and kernels.
#pragma once

#include <stdint.h>

#include "layout.h"

namespace bsk {

constexpr int kWave = 64;
constexpr int kMaxPages = 1024;  // page ids one work item may stage in LDS

// Launch arguments of the attention kernels.  They depend only on the
// problem, the tensors and the workspace addresses -- never on the plan's
// contents -- so one capture of a launch stays valid across plans.
struct AttnArgs {
  const void* q;
  int64_t q_st, q_sh;
  const void* k;
  const void* v;
  int64_t k_sp, k_sh, k_st;
  int64_t v_sp, v_sh, v_st;
  const int32_t* page_indices;
  void* out;
  int64_t o_st, o_sh;
  float* lse;
  int64_t lse_st;
  float* part_o;    // [slots][tile_q][D]
  float* part_lse;  // [slots][tile_q]
  const int32_t* ws;
  int32_t* ws_rw;     // same buffer: the arrival counters are updated in place
  const float* rope;  // [n_pos][D/2][2]
  int32_t rope_n_pos;
  int32_t group;
  int32_t page_shift;
  int32_t causal;
  int32_t window;
  int32_t sink;
  int32_t out_bf16;
  int32_t fused_merge;  // 1: the chunk that completes a split unit merges it in-kernel
  float scale_log2;     // sm_scale * log2(e): logits are kept in base 2
  // shared dense prefix of a composable batch (class-2 items of the mixed launch)
  const void* pk;
  const void* pv;
  int64_t pk_st, pk_sh, pv_st, pv_sh;
};

// Launch arguments of the append kernel (new tokens' K/V into the paged cache).
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  int64_t new_st, new_sh;  // token / head strides (elements) of k_new and v_new
  void* k_cache;
  void* v_cache;
  int64_t k_sp, k_sh, k_st;
  int64_t v_sp, v_sh, v_st;
  const int32_t* append_indptr;  // [batch + 1] new-token offsets (device)
  const int32_t* kv_len;         // [batch] lengths after the append (device)
  const int32_t* page_indptr;    // [batch + 1] page-list offsets (device)
  const int32_t* page_indices;   // page lists (device)
  int32_t batch;
  int32_t n_total;
  int32_t num_kv_heads;
  int32_t page_shift;
};

// Launch arguments of the unfused RoPE pass (rotated visible keys and query into scratch).
struct RopeApplyArgs {
  const void* q;
  int64_t q_st, q_sh;
  void* q_out;
  int64_t qo_st, qo_sh;
  const void* k;
  void* k_out;  // same strides as k
  int64_t k_sp, k_sh, k_st;
  const int32_t* qo_indptr;     // [batch + 1] (device)
  const int32_t* kv_len;        // [batch] (device)
  const int32_t* page_indptr;   // [batch + 1] (device)
  const int32_t* page_indices;  // (device)
  const float* rope;            // [n_pos][D/2][2]
  int32_t rope_n_pos;
  int32_t batch;
  int32_t num_qo_heads, num_kv_heads;
  int32_t page_shift;
  int32_t window, sink;
  int32_t streaming;  // 1: rank in the visible set, 0: token index
};

struct MergeArgs {
  const int32_t* ws;
  const float* part_o;
  const float* part_lse;
  void* out;
  int64_t o_st, o_sh;
  float* lse;
  int64_t lse_st;
  int32_t group;
  int32_t out_bf16;
};

}  // namespace bsk
