// Small-tile persistent attention kernel: one workgroup per worker walks its
// item list; the per-item work is decode_item (decode_item.h).

#include "decode_item.h"
#include "launch.h"

namespace bsk {

template <typename T, int D, bool DENSE, int ROPE, bool SAME>
__global__ __launch_bounds__(kDecThreads, ROPE == ROPE_NONE ? 3 : 2) void decode_kernel(AttnArgs a) {
  __shared__ __align__(16) DecodeSmem<D> s_dec;
  __shared__ int32_t s_pages[DENSE ? 1 : kMaxPages];
  __shared__ int s_last;
  const int32_t* __restrict__ ws = a.ws;
  const int it_begin = ws[HDR_WORDS + blockIdx.x];
  const int it_end = ws[HDR_WORDS + blockIdx.x + 1];
  const int32_t* __restrict__ items = ws + ws[HDR_OFF_ITEMS];
  for (int it = it_begin; it < it_end; ++it)
    decode_item<T, D, DENSE, ROPE, SAME>(a, items + int64_t(it) * ITEM_WORDS, s_dec, s_pages, &s_last, kDecRows);
}

// ---------------------------------------------------------------- host launchers

template <typename T, int D, bool DENSE, int ROPE, bool SAME>
hipError_t launch_one(const AttnArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<T, D, DENSE, ROPE, SAME>), dim3(grid), dim3(kDecThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, bool DENSE, int ROPE, bool SAME>
const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&decode_kernel<T, D, DENSE, ROPE, SAME>);
}

// (element type, head_dim, dense KV, RoPE mode, equal K/V strides); f32 is built with
// independent strides only
#define BSK_DEC_VARIANTS(X)                    \
  X(__bf16, 128, false, ROPE_NONE, true)       \
  X(__bf16, 128, true, ROPE_NONE, true)        \
  X(__bf16, 64, false, ROPE_NONE, true)        \
  X(__bf16, 64, true, ROPE_NONE, true)         \
  X(__bf16, 128, false, ROPE_STREAMING, true)  \
  X(__bf16, 128, false, ROPE_ABSOLUTE, true)   \
  X(__bf16, 64, false, ROPE_STREAMING, true)   \
  X(__bf16, 64, false, ROPE_ABSOLUTE, true)    \
  X(__bf16, 128, false, ROPE_NONE, false)      \
  X(__bf16, 128, true, ROPE_NONE, false)       \
  X(__bf16, 64, false, ROPE_NONE, false)       \
  X(__bf16, 64, true, ROPE_NONE, false)        \
  X(__bf16, 128, false, ROPE_STREAMING, false) \
  X(__bf16, 128, false, ROPE_ABSOLUTE, false)  \
  X(__bf16, 64, false, ROPE_STREAMING, false)  \
  X(__bf16, 64, false, ROPE_ABSOLUTE, false)   \
  X(float, 64, false, ROPE_NONE, false)        \
  X(float, 64, true, ROPE_NONE, false)         \
  X(float, 128, false, ROPE_NONE, false)       \
  X(float, 128, true, ROPE_NONE, false)

// dtype: 0 f32, 1 bf16.  same: K and V strides are equal (ignored for f32).  Returns
// hipErrorInvalidValue for combinations not built.
hipError_t launch_decode(int dtype, int head_dim, bool dense, int rope, bool same, const AttnArgs& a, int grid,
                         hipStream_t stream) {
  if (dtype == 0) same = false;
#define BSK_DEC(T, D, DN, R, S)                                                                        \
  if ((dtype == 1) == __is_same(T, __bf16) && head_dim == D && dense == DN && rope == R && same == S) \
    return launch_one<T, D, DN, R, S>(a, grid, stream);
  BSK_DEC_VARIANTS(BSK_DEC)
#undef BSK_DEC
  return hipErrorInvalidValue;
}

const void* decode_kernel_ptr(int dtype, int head_dim, bool dense, int rope, bool same) {
  if (dtype == 0) same = false;
#define BSK_DEC(T, D, DN, R, S)                                                                        \
  if ((dtype == 1) == __is_same(T, __bf16) && head_dim == D && dense == DN && rope == R && same == S) \
    return kernel_ptr<T, D, DN, R, S>();
  BSK_DEC_VARIANTS(BSK_DEC)
#undef BSK_DEC
  return nullptr;
}

int decode_threads() { return kDecThreads; }

}  // namespace bsk
