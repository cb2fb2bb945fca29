// Unfused RoPE: rotate the keys a decode query will see (and the query) ahead of a plain
// attention pass.
//
// The fused decode rotates each key as it streams it from HBM (FlashInfer
// paper summary, "Results": the fused RoPE + attention kernel).  This kernel
// is the unfused reference point for that comparison: for every request it
// rotates the visible keys -- the sliding window plus the attention sinks
// (FlashInfer 0.6 wiki, "Kernel types": the GQA decode with sliding window
// and sinks) -- into a scratch K pool at the same page slots, and rotates the
// request's query, so that attention without RoPE over (scratch K, original
// V) gives the RoPE result.  Positions are the streaming ranks (rank in the
// visible set, the query last) or the token indices.  Rotate-half form with
// the fp32 cos/sin table of bsk_rope_table; computed in fp32, stored in the
// cache's bf16.  HBM-bound: each visible key is read and written once.

#include "device.h"
#include "launch.h"

namespace bsk {

constexpr int kRopeThreads = 256;
constexpr int kRopeKeysPerBlock = 64;

// Rotate one pair of 8-element bf16 pieces (columns 8c.. and D/2 + 8c..) by the table row cs.
__device__ __forceinline__ void rope_pair(const __bf16* src, __bf16* dst, int c, int half,
                                          const float* __restrict__ cs) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(src + 8 * c);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(src + half + 8 * c);
  const float4* c4 = reinterpret_cast<const float4*>(cs + 16 * c);  // (cos, sin) of frequencies 8c..8c+7
  u32x4 olo, ohi;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float4 t = c4[w];  // cos_e, sin_e, cos_e+1, sin_e+1 for e = 8c + 2w
    const float x0 = bf16_lo(lo[w]), x1 = bf16_hi(lo[w]);
    const float y0 = bf16_lo(hi[w]), y1 = bf16_hi(hi[w]);
    olo[w] = pack_bf16x2(x0 * t.x - y0 * t.y, x1 * t.z - y1 * t.w);
    ohi[w] = pack_bf16x2(y0 * t.x + x0 * t.y, y1 * t.z + x1 * t.w);
  }
  *reinterpret_cast<u32x4*>(dst + 8 * c) = olo;
  *reinterpret_cast<u32x4*>(dst + half + 8 * c) = ohi;
}

template <int D>
__global__ __launch_bounds__(kRopeThreads) void rope_apply_kernel(RopeApplyArgs a) {
  constexpr int HALF = D / 2;
  constexpr int PAIRS = D / 16;  // 8-element piece pairs per head row
  const int r = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int L = a.kv_len[r];
  if (L <= 0) return;
  const int qpos = L - 1;  // one query per request: the last token
  const int lo_w = a.window > 0 ? max(0, qpos - a.window + 1) : 0;
  const int n_s = a.window > 0 ? min(a.sink, lo_w) : 0;
  const int n_vis = n_s + (L - lo_w);
  const __bf16* K = static_cast<const __bf16*>(a.k);
  __bf16* Ko = static_cast<__bf16*>(a.k_out);
  const int pairs = a.num_kv_heads * PAIRS;

  if (blockIdx.x == 0) {  // the query's rows (all q heads)
    const int tok = a.qo_indptr[r + 1] - 1;
    if (tok >= a.qo_indptr[r]) {
      const int pq = min(a.streaming ? n_vis - 1 : qpos, a.rope_n_pos - 1);
      const __bf16* Q = static_cast<const __bf16*>(a.q);
      __bf16* Qo = static_cast<__bf16*>(a.q_out);
      for (int e = threadIdx.x; e < a.num_qo_heads * PAIRS; e += kRopeThreads) {
        const int hq = e / PAIRS, c = e % PAIRS;
        rope_pair(Q + int64_t(tok) * a.q_st + int64_t(hq) * a.q_sh,
                  Qo + int64_t(tok) * a.qo_st + int64_t(hq) * a.qo_sh, c, HALF,
                  a.rope + int64_t(pq) * D);
      }
    }
  }

  const int v0 = blockIdx.x * kRopeKeysPerBlock;
  const int v1 = min(v0 + kRopeKeysPerBlock, n_vis);
  for (int v = v0 + wave; v < v1; v += kRopeThreads / kWave) {  // one wave per visible key
    const int t = v < n_s ? v : lo_w + (v - n_s);
    const int pk = min(a.streaming ? v : t, a.rope_n_pos - 1);
    const int64_t page = a.page_indices[int64_t(a.page_indptr[r]) + (t >> a.page_shift)];
    const int64_t slot = t & ((1 << a.page_shift) - 1);
    for (int p = lane; p < pairs; p += kWave) {
      const int h = p / PAIRS, c = p % PAIRS;
      const int64_t off = page * a.k_sp + int64_t(h) * a.k_sh + slot * a.k_st;
      rope_pair(K + off, Ko + off, c, HALF, a.rope + int64_t(pk) * D);
    }
  }
}

hipError_t launch_rope_apply(int head_dim, const RopeApplyArgs& a, int max_visible, hipStream_t stream) {
  const dim3 grid((max_visible + kRopeKeysPerBlock - 1) / kRopeKeysPerBlock > 0
                      ? (max_visible + kRopeKeysPerBlock - 1) / kRopeKeysPerBlock
                      : 1,
                  a.batch);
  if (head_dim == 128)
    hipLaunchKernelGGL(rope_apply_kernel<128>, grid, dim3(kRopeThreads), 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(rope_apply_kernel<64>, grid, dim3(kRopeThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bsk
