// Append of new tokens' K and V into the paged cache.
//
// Chunked prefill writes a chunk's new tokens after the cached ones and then
// attends over the whole sequence (FlashInfer 0.6 wiki, "Kernel types":
// Prefill).  New token i of request r becomes the last-but-(n_r - 1 - i)
// token of its sequence: logical position kv_len[r] - n_r + i, i.e. page
// kv_page_indices[kv_page_indptr[r] + pos / page_size], slot pos % page_size
// of the block-sparse layout (FlashInfer paper summary, "Research
// methodology" 1).  A pure copy: one wave per token finds the token's request
// with a wave-uniform binary search and moves the token's K and V rows (all
// kv heads) in 16-byte pieces.  HBM-bound: 2 (K, V) x Hk x d x element size
// bytes read and written per token.

#include "device.h"
#include "launch.h"

namespace bsk {

constexpr int kAppendThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  constexpr int PIECES = D * int(sizeof(T)) / 16;  // 16-byte pieces per head row
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int waves = gridDim.x * (kAppendThreads / kWave);
  const int pieces = a.num_kv_heads * PIECES;
  const char* kn = static_cast<const char*>(a.k_new);
  const char* vn = static_cast<const char*>(a.v_new);
  char* kc = static_cast<char*>(a.k_cache);
  char* vc = static_cast<char*>(a.v_cache);
  for (int t = blockIdx.x * (kAppendThreads / kWave) + wave; t < a.n_total; t += waves) {
    // request of token t: largest r with append_indptr[r] <= t (empty requests are skipped)
    int lo = 0, hi = a.batch;  // invariant: append_indptr[lo] <= t < append_indptr[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.append_indptr[mid] <= t) lo = mid; else hi = mid;
    }
    const int r = lo;
    const int n_r = a.append_indptr[r + 1] - a.append_indptr[r];
    const int pos = a.kv_len[r] - n_r + (t - a.append_indptr[r]);
    if (pos < 0) continue;  // kv_len shorter than the new tokens: nothing valid to write
    const int64_t slot_idx = int64_t(a.page_indptr[r]) + (pos >> a.page_shift);
    if (slot_idx >= a.page_indptr[r + 1]) continue;  // past the request's page list
    const int64_t page = a.page_indices[slot_idx];
    const int64_t in_page = pos & ((1 << a.page_shift) - 1);
    for (int p = lane; p < pieces; p += kWave) {
      const int h = p / PIECES, c = p % PIECES;
      const int64_t src_k = (int64_t(t) * a.new_st + int64_t(h) * a.new_sh) * int64_t(sizeof(T)) + 16 * c;
      const int64_t src_v = src_k;
      const int64_t dst_k = (page * a.k_sp + int64_t(h) * a.k_sh + in_page * a.k_st) * int64_t(sizeof(T)) + 16 * c;
      const int64_t dst_v = (page * a.v_sp + int64_t(h) * a.v_sh + in_page * a.v_st) * int64_t(sizeof(T)) + 16 * c;
      const u32x4 kx = *reinterpret_cast<const u32x4*>(kn + src_k);
      const u32x4 vx = *reinterpret_cast<const u32x4*>(vn + src_v);
      *reinterpret_cast<u32x4*>(kc + dst_k) = kx;
      *reinterpret_cast<u32x4*>(vc + dst_v) = vx;
    }
  }
}

hipError_t launch_append(int dtype, int head_dim, const AppendArgs& a, hipStream_t stream) {
  const int per_block = kAppendThreads / kWave;
  const int64_t want = (int64_t(a.n_total) + per_block - 1) / per_block;
  const int grid = int(want < 8192 ? (want > 0 ? want : 1) : 8192);
  if (dtype == 1 && head_dim == 128)
    hipLaunchKernelGGL((append_kernel<__bf16, 128>), dim3(grid), dim3(kAppendThreads), 0, stream, a);
  else if (dtype == 1 && head_dim == 64)
    hipLaunchKernelGGL((append_kernel<__bf16, 64>), dim3(grid), dim3(kAppendThreads), 0, stream, a);
  else if (dtype == 0 && head_dim == 128)
    hipLaunchKernelGGL((append_kernel<float, 128>), dim3(grid), dim3(kAppendThreads), 0, stream, a);
  else if (dtype == 0 && head_dim == 64)
    hipLaunchKernelGGL((append_kernel<float, 64>), dim3(grid), dim3(kAppendThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bsk
