// Large-tile persistent attention kernels: one workgroup per worker walks its
// item list; the per-item work is prefill_item (prefill_item.h), 32 query rows
// per wave: 128-row items on four-wave workgroups (two per CU) and 256-row
// items on eight-wave workgroups (one per CU, the same two waves per SIMD).
// The eight waves of a 256-row item share every K/V tile staged in LDS, so a
// tile serves twice the rows for the same transfers; each wave runs freely
// between the per-tile barriers.  The item body takes the logit max with
// fmaxf on values that are never NaN, so this file is built without NaN
// semantics.

#include "launch.h"
#include "prefill_item.h"

namespace bsk {

// WAVES = 4: 128-row items, two workgroups per CU.  WAVES = 8: 256-row items, one per CU.
template <int D, bool DENSE, int WAVES, bool SAME>
__global__ __launch_bounds__(WAVES * kWave, WAVES == 4 ? 2 : 1) void prefill_kernel(AttnArgs a) {
  __shared__ __align__(1024) PrefillSmem<D> s_pre;
  __shared__ int32_t s_pages[DENSE ? 1 : kMaxPages];
  __shared__ int s_last;
  const int32_t* __restrict__ ws = a.ws;
  const int it_begin = ws[HDR_WORDS + blockIdx.x];
  const int it_end = ws[HDR_WORDS + blockIdx.x + 1];
  const int32_t* __restrict__ items = ws + ws[HDR_OFF_ITEMS];
  for (int it = it_begin; it < it_end; ++it)
    prefill_item<D, DENSE, 2, SAME, WAVES>(a, items + int64_t(it) * ITEM_WORDS, s_pre, s_pages, &s_last);
}

// (head_dim, dense KV, waves per workgroup, equal K/V strides); tile_q = 32 * waves
#define BSK_PRE_VARIANTS(X) \
  X(128, false, 4, true)    \
  X(128, true, 4, true)     \
  X(64, false, 4, true)     \
  X(64, true, 4, true)      \
  X(128, false, 8, true)    \
  X(128, true, 8, true)     \
  X(64, false, 8, true)     \
  X(64, true, 8, true)      \
  X(128, false, 4, false)   \
  X(128, true, 4, false)    \
  X(64, false, 4, false)    \
  X(64, true, 4, false)     \
  X(128, false, 8, false)   \
  X(128, true, 8, false)    \
  X(64, false, 8, false)    \
  X(64, true, 8, false)

hipError_t launch_prefill(int head_dim, bool dense, int tile_q, bool same, const AttnArgs& a, int grid,
                          hipStream_t stream) {
#define BSK_PRE(D, DN, WV, S)                                                                         \
  if (head_dim == D && dense == DN && tile_q == 32 * WV && same == S) {                               \
    hipLaunchKernelGGL((prefill_kernel<D, DN, WV, S>), dim3(grid), dim3(WV * kWave), 0, stream, a); \
    return hipGetLastError();                                                                         \
  }
  BSK_PRE_VARIANTS(BSK_PRE)
#undef BSK_PRE
  return hipErrorInvalidValue;
}

const void* prefill_kernel_ptr(int head_dim, bool dense, int tile_q, bool same) {
#define BSK_PRE_PTR(D, DN, WV, S)                                      \
  if (head_dim == D && dense == DN && tile_q == 32 * WV && same == S) \
    return reinterpret_cast<const void*>(&prefill_kernel<D, DN, WV, S>);
  BSK_PRE_VARIANTS(BSK_PRE_PTR)
#undef BSK_PRE_PTR
  return nullptr;
}

int prefill_threads(int tile_q) { return tile_q == 256 ? 8 * kWave : kPreThreads; }

}  // namespace bsk
