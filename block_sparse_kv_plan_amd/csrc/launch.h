// Host-side launchers of the device kernels (defined in the .hip files).
#pragma once

#include <hip/hip_runtime.h>

#include "args.h"

namespace bsk {

hipError_t launch_decode(int dtype, int head_dim, bool dense, int rope, bool same, const AttnArgs& a, int grid,
                         hipStream_t stream);
const void* decode_kernel_ptr(int dtype, int head_dim, bool dense, int rope, bool same);
int decode_threads();

hipError_t launch_prefill(int head_dim, bool dense, int tile_q, bool same, const AttnArgs& a, int grid,
                          hipStream_t stream);
const void* prefill_kernel_ptr(int head_dim, bool dense, int tile_q, bool same);
int prefill_threads(int tile_q);

hipError_t launch_mixed(int head_dim, bool same, const AttnArgs& a, int grid, hipStream_t stream);
const void* mixed_kernel_ptr(int head_dim, bool same);

hipError_t launch_rope_apply(int head_dim, const RopeApplyArgs& a, int max_visible, hipStream_t stream);
hipError_t launch_append(int dtype, int head_dim, const AppendArgs& a, hipStream_t stream);

hipError_t launch_merge(int head_dim, const MergeArgs& a, int grid, hipStream_t stream);
hipError_t launch_merge_pair(const float* oa, const float* la, const float* ob, const float* lb, void* out,
                             float* lse_out, int rows, int D, int out_bf16, hipStream_t stream);
// Copies `words` 32-bit words from a pinned host buffer's device address into device memory, on
// `stream`; both pointers 16-byte aligned.
hipError_t launch_plan_upload(const void* src_dev, void* dst, int64_t words, hipStream_t stream);
// The merge (grid `merge_grid`) and a plan upload into another workspace in one launch.
hipError_t launch_merge_upload(int head_dim, const MergeArgs& a, int merge_grid, const void* src_dev, void* dst,
                               int64_t words, hipStream_t stream);
hipError_t launch_rope_table(float* table, int n_pos, int D, double theta, hipStream_t stream);
// Device address and size of the no-allocation scratch array on the current device (looked up on
// the first call per device).
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// Reads n16 16-byte pieces of src once; sink gets one word per thread (grid * stream_read_threads()).
hipError_t launch_stream_read(const void* src, int64_t n16, uint32_t* sink, int grid, hipStream_t stream);
int stream_read_threads();
hipError_t launch_block_read(const void* src, int64_t n_buf_blocks, const int32_t* order, int32_t n_blocks,
                             uint32_t* sink, int grid, hipStream_t stream);

hipError_t launch_gather(int dtype, int head_dim, bool dense, const AttnArgs& a, const int64_t* row_off, void* k_out,
                         void* v_out, int grid, hipStream_t stream);

}  // namespace bsk
