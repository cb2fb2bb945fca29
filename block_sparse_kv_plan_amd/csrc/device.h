// Device-side helpers shared by the attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (lo in bits 0..15), round-to-nearest-even;
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// acc + lo + hi of a packed bf16 pair, in fp32 (one v_dot2c_f32_bf16 against (1, 1)): the sum of
// probabilities exactly as the PV product sees them once they are rounded to bf16.
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  const bf16x2_t one = {__bf16(1.0f), __bf16(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}

// Partial states exchanged inside one launch (the in-kernel merge) pass between workgroups that
// may run on different XCDs, whose L2 caches are not coherent with each other.  They are stored
// and loaded as relaxed device-scope atomics (cache-coherent accesses at the device's coherence
// point), so publishing them needs only the wait for the stores to complete -- no L2 writeback
// or invalidation.  Without the in-kernel merge they are plain accesses.
__device__ __forceinline__ void store_part(float* p, float v, bool coherent) {
  if (coherent)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
__device__ __forceinline__ void store_part4(float* p, float x, float y, float z, float w, bool coherent) {
  if (coherent) {
    store_part(p, x, true);
    store_part(p + 1, y, true);
    store_part(p + 2, z, true);
    store_part(p + 3, w, true);
  } else {
    *reinterpret_cast<float4*>(p) = float4{x, y, z, w};
  }
}
template <bool COHERENT>
__device__ __forceinline__ float load_part(const float* p) {
  if constexpr (COHERENT)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}
template <bool COHERENT>
__device__ __forceinline__ float4 load_part4(const float* p) {
  if constexpr (COHERENT)
    return float4{load_part<true>(p), load_part<true>(p + 1), load_part<true>(p + 2), load_part<true>(p + 3)};
  else
    return *reinterpret_cast<const float4*>(p);
}

// Merge of one (row, 4 columns) of a split unit from its chunks' partial
// states: M = max_c LSE_c, w_c = exp(LSE_c - M), O = sum_c w_c O_c / sum_c w_c,
// LSE = M + ln sum_c w_c; every chunk empty gives O = 0, LSE = -inf.  Writes
// the output row (and the LSE when c4 == 0).  With a shared prefix
// (rec[MG_PFX_N] > 0) the row's prefix partials join the chunks: the row is
// global query row R = q0 * g + row_lo + rr, held as row R % tile_q of the
// prefix tile R / tile_q of its kv head.
template <int D, bool COHERENT = false>
__device__ __forceinline__ void merge_row(const int32_t* rec, int rr, int c4, int tile_q,
                                          const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                          int q0, int g, void* out, int64_t o_st, int64_t o_sh, float* lse_out,
                                          int64_t lse_st, int out_bf16) {
  const int h = rec[MG_H], row_lo = rec[MG_ROW_LO];
  const int first = rec[MG_FIRST_SLOT], n_own = rec[MG_N], n_pfx = rec[MG_PFX_N];
  const int nc = n_own + n_pfx;
  // partial-state rows (slot * tile_q + row) of the row's own chunks and of its prefix chunks
  const int64_t own0 = int64_t(first) * tile_q + rr;
  const int64_t R = int64_t(q0) * g + row_lo + rr;
  const int64_t pfx0 = n_pfx > 0 ? (int64_t(rec[MG_PFX_FIRST]) + (R / tile_q) * n_pfx) * tile_q + R % tile_q : 0;
  auto part_row = [&](int c) { return c < n_own ? own0 + int64_t(c) * tile_q : pfx0 + int64_t(c - n_own) * tile_q; };
  // chunks in groups of eight: all loads of a group are issued together (one memory latency per
  // group), then the group's maximum moves the running reference and its terms are added
  float M = -INFINITY, wsum = 0.f;
  float4 o = {0, 0, 0, 0};
  for (int c0 = 0; c0 < nc; c0 += 8) {
    float lc[8];
    float4 x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // past the last chunk: the last chunk's values are read again (always in bounds, so the
      // loads need no predicate) and weighted 0
      const int64_t pr = part_row(min(c0 + k, nc - 1));
      const float l = load_part<COHERENT>(part_lse + pr);
      lc[k] = c0 + k < nc ? l : -INFINITY;
      x[k] = load_part4<COHERENT>(part_o + pr * D + c4);
    }
    float gm = lc[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) gm = fmaxf(gm, lc[k]);
    if (gm > M) {
      const float sc = __expf(M - gm);  // 0 while M is still -inf
      o.x *= sc;
      o.y *= sc;
      o.z *= sc;
      o.w *= sc;
      wsum *= sc;
      M = gm;
    }
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float w = lc[k] == -INFINITY ? 0.f : __expf(lc[k] - M);  // an empty chunk holds O = 0
        o.x += w * x[k].x;
        o.y += w * x[k].y;
        o.z += w * x[k].z;
        o.w += w * x[k].w;
        wsum += w;
      }
    }
  }
  float lse = -INFINITY;
  if (wsum > 0.f) {
    const float inv = 1.f / wsum;
    o.x *= inv;
    o.y *= inv;
    o.z *= inv;
    o.w *= inv;
    lse = M + __logf(wsum);
  }
  const int row = row_lo + rr;
  const int tok = q0 + row / g;
  const int qhd = h * g + row % g;
  const int64_t oo = int64_t(tok) * o_st + int64_t(qhd) * o_sh + c4;
  if (out_bf16) {
    uint2 pk2 = {pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
    *reinterpret_cast<uint2*>(static_cast<__bf16*>(out) + oo) = pk2;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + oo) = o;
  }
  if (c4 == 0) lse_out[int64_t(tok) * lse_st + qhd] = lse;
}

// Called by all threads of a workgroup right after they stored one chunk's
// partial state (slot `slot`).  Publishes the partial, counts the chunk in
// the unit's arrival counter, and if this was the unit's last chunk merges
// the unit in place and resets the counter for the next run.
template <int D>
__device__ __forceinline__ void finish_split_chunk(const AttnArgs& a, int slot, int tid, int nthreads,
                                                   int* s_flag) {
  const int32_t* __restrict__ ws = a.ws;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial-state stores have completed (device-coherent)
  __syncthreads();
  const int m = ws[ws[HDR_OFF_SLOTMAP] + slot];
  const int32_t* rec = ws + ws[HDR_OFF_MERGE] + int64_t(m) * MERGE_WORDS;
  if (tid == 0) {
    int32_t* cnt = a.ws_rw + ws[HDR_OFF_COUNT] + m;
    const int prev = atomicAdd(cnt, 1);
    const int last = prev == rec[MG_N] - 1;
    if (last) atomicExch(cnt, 0);
    *s_flag = last;
  }
  __syncthreads();
  if (*s_flag) {
    // the other chunks' partial states are read with device-coherent loads, issued only now
    const int tile_q = ws[HDR_TILE_Q];
    const int q0 = (ws + ws[HDR_OFF_QO])[rec[MG_R]];
    const int nrows = rec[MG_ROW_HI] - rec[MG_ROW_LO];
    for (int e = tid; e < nrows * (D / 4); e += nthreads)
      merge_row<D, true>(rec, e / (D / 4), (e % (D / 4)) * 4, tile_q, a.part_o, a.part_lse, q0, a.group, a.out,
                         a.o_st, a.o_sh, a.lse, a.lse_st, a.out_bf16);
  }
  __syncthreads();
}

// Visible keys of one query row as integer bounds, so that each key's test
// is a few compares and a select (no per-key branches): key t is visible iff
// t < hi and (t >= lo or t < sink_hi).  Keys past the item's range, the
// causal bound and the sliding window (with its sinks) fold into the bounds;
// a row outside the tile sees nothing.
struct RowMask {
  int lo, hi, sink_hi;
};

__device__ __forceinline__ RowMask row_mask(bool row_ok, int qpos, int kv_hi, int causal, int window, int sink) {
  RowMask m;
  m.hi = row_ok ? (causal ? min(kv_hi, qpos + 1) : kv_hi) : INT_MIN;
  m.lo = window > 0 ? qpos - window + 1 : INT_MIN;
  m.sink_hi = window > 0 ? sink : INT_MIN;
  return m;
}

__device__ __forceinline__ bool row_sees(const RowMask& m, int t) {
  return (t < m.hi) & ((t >= m.lo) | (t < m.sink_hi));
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

// LDS byte address of a shared-memory location.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}

// Direct global-to-LDS transfers: lane l's 16 (4) bytes at g land at LDS byte lds + 16 l
// (lds + 4 l), lds wave-uniform.  Written as inline assembly so that the compiler adds no waits
// of its own; completion is tracked by vmcnt only and the caller waits (wait_vm) before the
// barrier that publishes the data.  Nothing else in these kernels relies on m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(0) (expcnt, lgkmcnt unconstrained) as a real instruction the compiler's wait
// bookkeeping sees: after it no vector-memory load of this wave is outstanding, so the compiler
// places no further vmcnt wait in front of uses of earlier loads (which would also stall on the
// next tile's transfers).
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_dma() {
  asm volatile("" ::: "memory");
  wait_vm();
}

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
