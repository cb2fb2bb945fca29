// Host work planner (no HIP dependency; builds with a plain C++17 compiler).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

namespace bsk {

struct PlanParams {
  int32_t num_qo_heads = 0;
  int32_t num_kv_heads = 0;
  int32_t tile_q = 0;
  int32_t tile_kv = 0;
  int32_t num_workers = 0;
  int32_t split_factor = 1;
  int32_t min_chunk = 0;
  int32_t max_chunk = 0;
  int32_t item_overhead = 0;
  int32_t max_batch = 0;
  int32_t max_items_per_worker = 0;
  int32_t max_slots = 0;
  int32_t max_merge = 0;
  bool causal = false;
  int32_t window = 0;
  int32_t sink = 0;
  int32_t decode_tile_q = 0;  // > 0: requests with qo_len * g <= decode_tile_q get one decode-class tile
  int32_t shared_prefix_len = 0;  // > 0: a dense prefix of this many tokens shared by every request
};

struct PlanStats {
  int32_t num_items = 0;
  int32_t num_slots = 0;
  int32_t num_merge = 0;
  int32_t chunk = 0;
  int32_t max_kv_len = 0;
  int32_t max_qo_len = 0;
  int32_t max_items_on_worker = 0;
  int64_t total_cost = 0;
  int64_t max_load = 0;
  int64_t used_bytes = 0;
};

enum PlanResult { PLAN_OK = 0, PLAN_INVALID = -1, PLAN_CAPACITY = -3, PLAN_WORKSPACE = -4 };

// Capacity (bytes) of the int workspace for these parameters.
size_t plan_workspace_bytes(const PlanParams& p);

// Build the plan into `buf` (capacity `buf_bytes`).  `kv_indptr` is copied
// through unchanged for the kernels.  On failure `err` says why.
PlanResult build_plan(const PlanParams& p, int32_t batch, const int32_t* qo_indptr, const int32_t* kv_len,
                      const int32_t* kv_indptr, int32_t* buf, size_t buf_bytes, PlanStats* stats,
                      std::string* err);

}  // namespace bsk
