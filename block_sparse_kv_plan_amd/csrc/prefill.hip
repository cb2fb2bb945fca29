// Large-tile persistent attention kernels: one workgroup per worker walks its
// item list; the per-item work is prefill_item (128-row items, four waves,
// prefill_item.h) or prefill_pp_item (256-row items, eight waves in two
// alternating groups, prefill_pp_item.h).  The item bodies take the logit
// max with fmaxf on values that are never NaN, so this file is built without
// NaN semantics.

#include <type_traits>

#include "launch.h"
#include "prefill_pp_item.h"

namespace bsk {

// NB = 2: 128-row items, two workgroups per CU.  NB = 4: 256-row items, eight waves.
template <int NB>
constexpr int pre_threads() {
  return NB == 2 ? kPreThreads : kPPThreads;
}

template <int D, int NB>
using PreSmem = typename std::conditional<NB == 2, PrefillSmem<D>, PrefillPPSmem<D>>::type;

template <int D, bool DENSE, int NB, bool SAME>
__global__ __launch_bounds__(pre_threads<NB>(), NB == 2 ? 2 : 1) void prefill_kernel(AttnArgs a) {
  __shared__ __align__(1024) PreSmem<D, NB> s_pre;
  __shared__ int32_t s_pages[DENSE ? 1 : kMaxPages];
  __shared__ int s_last;
  const int32_t* __restrict__ ws = a.ws;
  const int it_begin = ws[HDR_WORDS + blockIdx.x];
  const int it_end = ws[HDR_WORDS + blockIdx.x + 1];
  const int32_t* __restrict__ items = ws + ws[HDR_OFF_ITEMS];
  for (int it = it_begin; it < it_end; ++it) {
    if constexpr (NB == 2)
      prefill_item<D, DENSE, 2, SAME>(a, items + int64_t(it) * ITEM_WORDS, s_pre, s_pages, &s_last);
    else
      prefill_pp_item<D, DENSE, SAME>(a, items + int64_t(it) * ITEM_WORDS, s_pre, s_pages, &s_last);
  }
}

#define BSK_PRE_VARIANTS(X) \
  X(128, false, 2, true)        \
  X(128, true, 2, true)         \
  X(64, false, 2, true)         \
  X(64, true, 2, true)          \
  X(128, false, 4, true)        \
  X(128, true, 4, true)         \
  X(64, false, 4, true)         \
  X(64, true, 4, true)          \
  X(128, false, 2, false)       \
  X(128, true, 2, false)        \
  X(64, false, 2, false)        \
  X(64, true, 2, false)         \
  X(128, false, 4, false)       \
  X(128, true, 4, false)        \
  X(64, false, 4, false)        \
  X(64, true, 4, false)

hipError_t launch_prefill(int head_dim, bool dense, int tile_q, bool same, const AttnArgs& a, int grid,
                          hipStream_t stream) {
#define BSK_PRE(D, DN, NB, S)                                                                          \
  if (head_dim == D && dense == DN && tile_q == 64 * NB && same == S) {                                \
    hipLaunchKernelGGL((prefill_kernel<D, DN, NB, S>), dim3(grid), dim3(pre_threads<NB>()), 0, stream, a); \
    return hipGetLastError();                                                                          \
  }
  BSK_PRE_VARIANTS(BSK_PRE)
#undef BSK_PRE
  return hipErrorInvalidValue;
}

const void* prefill_kernel_ptr(int head_dim, bool dense, int tile_q, bool same) {
#define BSK_PRE_PTR(D, DN, NB, S)                                      \
  if (head_dim == D && dense == DN && tile_q == 64 * NB && same == S) \
    return reinterpret_cast<const void*>(&prefill_kernel<D, DN, NB, S>);
  BSK_PRE_VARIANTS(BSK_PRE_PTR)
#undef BSK_PRE_PTR
  return nullptr;
}

int prefill_threads(int tile_q) { return tile_q == kPPRows ? kPPThreads : kPreThreads; }

}  // namespace bsk
