// One persistent launch over a mixed batch: decode-class and prefill-class
// work items on the same workers.
//
// A batch that holds both decode requests (one query token) and prefill
// requests (many) is planned as one set of work items in two tile classes
// (FlashInfer BatchAttention K/V stride optimisation, the analysis of PR
// #5329, "Code analysis" 1: one persistent kernel scheduling a decode-sized
// and a prefill-sized tile configuration together): a request
// whose qo_len * g rows fit one 16-row tile becomes small-tile items, every
// other request 128-row items, and the planner balances both over the same
// workers (FlashInfer paper summary, "Research methodology" 3).  Each
// workgroup walks its item list and runs each item with the body of its
// class -- decode_item or prefill_item, the same code as the single-class
// kernels -- so no request waits for a second launch.  The two bodies share
// one LDS allocation (a union); every item starts after a barrier, so an
// item never overwrites LDS that the previous one still reads.
//
// Partial states of split units are written with the plan's slot stride
// (the large tile, 128 rows) for both classes, so the merge (fused at the
// last chunk, or the separate merge pass) is the one of the large-tile plan.
// bf16, paged KV, no RoPE; 2 workgroups per CU (the prefill body's register
// and LDS budget).
//
// A composable batch (FlashInfer paper summary, "Research methodology" 1:
// a dense shared part and sparse per-request parts, each at its own block
// size) adds a third class: 128-row items of the dense prefix every request
// shares, over the batch's global query rows, run by the large-tile body on
// the prefix's own K/V.  Their partial states meet the suffix items' in the
// merge pass.

#include "decode_item.h"
#include "launch.h"
#include "prefill_item.h"

namespace bsk {

constexpr int kMixTileQ = 128;  // the large class: prefill_item with two row blocks per wave
static_assert(kDecThreads == kPreThreads, "both bodies run on the same workgroup shape");

template <int D>
union MixedSmem {
  DecodeSmem<D> dec;
  PrefillSmem<D> pre;
};

template <int D, bool SAME>
__global__ __launch_bounds__(kPreThreads, 2) void mixed_kernel(AttnArgs a) {
  __shared__ __align__(1024) MixedSmem<D> s_mix;
  __shared__ int32_t s_pages[kMaxPages];
  __shared__ int s_last;
  const int32_t* __restrict__ ws = a.ws;
  const int it_begin = ws[HDR_WORDS + blockIdx.x];
  const int it_end = ws[HDR_WORDS + blockIdx.x + 1];
  const int32_t* __restrict__ items = ws + ws[HDR_OFF_ITEMS];
  for (int it = it_begin; it < it_end; ++it) {
    const int32_t* rec = items + int64_t(it) * ITEM_WORDS;
    const int cls = rec[IT_CLASS];
    if (cls == 1) {
      __syncthreads();  // the previous item (either class) is done with the shared LDS
      decode_item<__bf16, D, false, ROPE_NONE, SAME>(a, rec, s_mix.dec, s_pages, &s_last, kMixTileQ);
    } else if (cls == 0) {
      prefill_item<D, false, kMixTileQ / 64, SAME, kPreWaves, false>(a, rec, s_mix.pre, s_pages, &s_last);  // opens with a barrier
    } else {
      // the shared dense prefix of a composable batch: the batch's global query rows against the
      // prefix's own K/V, every prefix key in every query's past (no mask)
      AttnArgs ap = a;
      ap.k = a.pk;
      ap.v = a.pv;
      ap.k_sp = 0;
      ap.v_sp = 0;
      ap.k_st = a.pk_st;
      ap.k_sh = a.pk_sh;
      ap.v_st = a.pv_st;
      ap.v_sh = a.pv_sh;
      ap.causal = 0;
      ap.window = 0;
      ap.sink = 0;
      prefill_item<D, true, kMixTileQ / 64, false, kPreWaves, false>(ap, rec, s_mix.pre, s_pages, &s_last);
    }
  }
}

#define BSK_MIX_VARIANTS(X) \
  X(128, true)              \
  X(64, true)               \
  X(128, false)             \
  X(64, false)

hipError_t launch_mixed(int head_dim, bool same, const AttnArgs& a, int grid, hipStream_t stream) {
#define BSK_MIX(D, S)                                                                            \
  if (head_dim == D && same == S) {                                                              \
    hipLaunchKernelGGL((mixed_kernel<D, S>), dim3(grid), dim3(kPreThreads), 0, stream, a);       \
    return hipGetLastError();                                                                    \
  }
  BSK_MIX_VARIANTS(BSK_MIX)
#undef BSK_MIX
  return hipErrorInvalidValue;
}

const void* mixed_kernel_ptr(int head_dim, bool same) {
#define BSK_MIX_PTR(D, S) \
  if (head_dim == D && same == S) return reinterpret_cast<const void*>(&mixed_kernel<D, S>);
  BSK_MIX_VARIANTS(BSK_MIX_PTR)
#undef BSK_MIX_PTR
  return nullptr;
}

}  // namespace bsk
