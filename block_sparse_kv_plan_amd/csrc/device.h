// Device-side helpers shared by the attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "args.h"

namespace bsk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Key visibility for a query at position qpos: causal, then sliding window
// or one of the first `sink` tokens.
__device__ __forceinline__ bool key_visible(int t, int qpos, int causal, int window, int sink) {
  bool ok = !causal || t <= qpos;
  if (window > 0) ok = ok && ((qpos - t) < window || t < sink);
  return ok;
}

__device__ __forceinline__ float wave_max_xor16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, kWave));
  x = fmaxf(x, __shfl_xor(x, 32, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum_xor16_32(float x) {
  x += __shfl_xor(x, 16, kWave);
  x += __shfl_xor(x, 32, kWave);
  return x;
}

}  // namespace bsk

namespace bsk {

// Block-sparse gather, part 1: stage the page ids an item needs -- pages
// kv_lo / page_size .. (kv_hi - 1) / page_size of request r's page list --
// into LDS, so every later key address is one LDS read away.  All threads
// of the workgroup take part; the caller synchronises afterwards.
__device__ __forceinline__ void stage_pages(int32_t* s_pages, const int32_t* __restrict__ page_indices,
                                            int kbase, int kv_lo, int kv_hi, int page_shift, int tid,
                                            int nthreads) {
  const int p0 = kv_lo >> page_shift;
  const int np = ((kv_hi - 1) >> page_shift) - p0 + 1;
  for (int i = tid; i < np; i += nthreads) s_pages[i] = page_indices[kbase + p0 + i];
}

// Block-sparse gather, part 2: element offset of key t (kv head h) of the
// item's request.  PAGED: page id from the staged list, then the slot in
// the page; DENSE: contiguous rows from the request's token offset.
template <bool DENSE>
__device__ __forceinline__ int64_t kv_offset(const int32_t* s_pages, int t, int kbase, int kv_lo, int page_shift,
                                             int h, int64_t sp, int64_t sh, int64_t st) {
  if constexpr (DENSE) {
    return int64_t(kbase + t) * st + int64_t(h) * sh;
  } else {
    const int page = s_pages[(t >> page_shift) - (kv_lo >> page_shift)];
    return int64_t(page) * sp + int64_t(h) * sh + int64_t(t & ((1 << page_shift) - 1)) * st;
  }
}

}  // namespace bsk
