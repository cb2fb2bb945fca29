// Partial-state merge, plan upload, RoPE table, the gather test hook and a streaming-read
// measurement hook.
//
// Split-KV (FlashInfer 0.6 wiki, "Kernel types": the split_kv decode path)
// leaves one (O_c, LSE_c) per key chunk; the exact combination is
//   M = max_c LSE_c,  LSE = M + ln sum_c exp(LSE_c - M),
//   O = sum_c exp(LSE_c - LSE) O_c,
// with every chunk empty (LSE_c = -inf) giving O = 0, LSE = -inf.  The
// composable format (FlashInfer paper summary, "Research methodology" 1)
// uses the same combination for a dense-prefix state and a paged-suffix
// state.

#include "device.h"
#include "launch.h"

namespace bsk {

constexpr int kMergeThreads = 256;

// Plan-driven merge: fixed grid.  Work is spread over (merge entry, row)
// pairs -- D/4 threads per row, each owning four columns -- so a few long
// entries (a prefix split into many chunks) still use the whole chip.  No
// entry has more rows than min(tile_q, longest query * group): decode entries
// (one token, a GQA group of rows) then take no idle threads.
template <int D>
__device__ __forceinline__ void merge_blocks(const MergeArgs& a, int block, int nblocks) {
  constexpr int TPR = D / 4;                  // threads per row
  constexpr int RPB = kMergeThreads / TPR;    // rows per block per pass
  const int32_t* __restrict__ ws = a.ws;
  const int n_merge = ws[HDR_NUM_MERGE];
  const int tile_q = ws[HDR_TILE_Q];
  const int rows = int(min(int64_t(tile_q), int64_t(ws[HDR_MAX_QO_LEN]) * a.group));
  const int32_t* __restrict__ table = ws + ws[HDR_OFF_MERGE];
  const int32_t* __restrict__ qo_indptr = ws + ws[HDR_OFF_QO];
  const int g = a.group;
  const int c4 = (threadIdx.x % TPR) * 4;
  const int64_t n_virtual = int64_t(n_merge) * rows;  // (entry, row) pairs
  for (int64_t v = int64_t(block) * RPB + threadIdx.x / TPR; v < n_virtual; v += int64_t(nblocks) * RPB) {
    const int m = int(v / rows);
    const int rr = int(v % rows);
    const int32_t* rec = table + int64_t(m) * MERGE_WORDS;
    if (rr >= rec[MG_ROW_HI] - rec[MG_ROW_LO]) continue;
    merge_row<D>(rec, rr, c4, tile_q, a.part_o, a.part_lse, qo_indptr[rec[MG_R]], g, a.out, a.o_st, a.o_sh, a.lse,
                 a.lse_st, a.out_bf16);
  }
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  merge_blocks<D>(a, blockIdx.x, gridDim.x);
}

// Row-wise merge of two complete states (composable prefix + suffix).
__global__ __launch_bounds__(kMergeThreads) void merge_pair_kernel(const float* __restrict__ oa,
                                                                   const float* __restrict__ la,
                                                                   const float* __restrict__ ob,
                                                                   const float* __restrict__ lb, void* out,
                                                                   float* lse_out, int rows, int D, int out_bf16) {
  const int per_row = D / 4;
  const int64_t total = int64_t(rows) * per_row;
  for (int64_t e = blockIdx.x * int64_t(kMergeThreads) + threadIdx.x; e < total;
       e += int64_t(gridDim.x) * kMergeThreads) {
    const int64_t row = e / per_row;
    const int c4 = int(e % per_row) * 4;
    const float x = la[row], y = lb[row];
    const float M = fmaxf(x, y);
    float4 o = {0, 0, 0, 0};
    float lse = -INFINITY;
    if (M != -INFINITY) {
      const float ex = __expf(x - M), ey = __expf(y - M);
      lse = M + __logf(ex + ey);
      const float wa = __expf(x - lse), wb = __expf(y - lse);
      const float4 p = *reinterpret_cast<const float4*>(oa + row * D + c4);
      const float4 q = *reinterpret_cast<const float4*>(ob + row * D + c4);
      o = float4{wa * p.x + wb * q.x, wa * p.y + wb * q.y, wa * p.z + wb * q.z, wa * p.w + wb * q.w};
    }
    if (out_bf16) {
      uint2 pk2 = {pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
      *reinterpret_cast<uint2*>(static_cast<__bf16*>(out) + row * D + c4) = pk2;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + row * D + c4) = o;
    }
    if (c4 == 0) lse_out[row] = lse;
  }
}

// table[p][k] = (cos, sin)(p * theta^(-2k/D)), evaluated in fp64.
__global__ void rope_table_kernel(float* table, int n_pos, int D, double theta) {
  const int half = D / 2;
  const int64_t total = int64_t(n_pos) * half;
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < total; e += int64_t(gridDim.x) * blockDim.x) {
    const int64_t p = e / half;
    const int k = int(e % half);
    const double inv_freq = pow(theta, -2.0 * double(k) / double(D));
    const double ang = double(p) * inv_freq;
    table[2 * e] = float(cos(ang));
    table[2 * e + 1] = float(sin(ang));
  }
}

// Test hook: copy every item's keys through the attention kernels' gather path.
template <typename T, int D, bool DENSE>
__global__ __launch_bounds__(256) void gather_kernel(AttnArgs a, const int64_t* __restrict__ row_off, T* kout,
                                                     T* vout) {
  __shared__ int32_t s_pages[DENSE ? 1 : kMaxPages];
  const int32_t* __restrict__ ws = a.ws;
  const int it_begin = ws[HDR_WORDS + blockIdx.x];
  const int it_end = ws[HDR_WORDS + blockIdx.x + 1];
  const int32_t* __restrict__ items = ws + ws[HDR_OFF_ITEMS];
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  for (int it = it_begin; it < it_end; ++it) {
    const int32_t* rec = items + int64_t(it) * ITEM_WORDS;
    const int h = rec[IT_H], kv_lo = rec[IT_KV_LO], kv_hi = rec[IT_KV_HI], id = rec[IT_ID];
    const int kbase = rec[IT_KBASE];
    if constexpr (!DENSE) stage_pages(s_pages, a.page_indices, kbase, kv_lo, kv_hi, a.page_shift, threadIdx.x, 256);
    __syncthreads();
    const int64_t base = row_off[id];
    for (int e = threadIdx.x; e < (kv_hi - kv_lo) * D; e += 256) {
      const int t = kv_lo + e / D;
      const int c = e % D;
      const int64_t ko = kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.k_sp, a.k_sh, a.k_st);
      const int64_t vo = kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.v_sp, a.v_sh, a.v_st);
      kout[(base + (t - kv_lo)) * D + c] = K[ko + c];
      vout[(base + (t - kv_lo)) * D + c] = V[vo + c];
    }
    __syncthreads();
  }
}

// Plan upload: the plan's words copied from the pinned host buffer (read through its device
// mapping) into the int workspace, by a kernel on the caller's stream.  Sixteen bytes per thread;
// both buffers are 16-byte aligned (the host checks), the last thread takes the ragged tail.
constexpr int kUploadWordsPerBlock = 256 * 4;

__device__ __forceinline__ void upload_block(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                             int64_t words, int block) {
  const int64_t i = (int64_t(block) * 256 + threadIdx.x) * 4;
  if (i + 4 <= words) {
    *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(src + i);
  } else {
    for (int64_t k = i; k < words; ++k) dst[k] = src[k];
  }
}

__global__ __launch_bounds__(256) void plan_upload_kernel(const uint32_t* __restrict__ src,
                                                          uint32_t* __restrict__ dst, int64_t words) {
  upload_block(src, dst, words, blockIdx.x);
}

// One launch for the merge of one plan's run and the upload of the next plan into another
// workspace (the two touch disjoint buffers): the first `upload_blocks` blocks copy the plan, the
// rest merge.  The upload then needs no dispatch of its own.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_upload_kernel(MergeArgs a, int upload_blocks,
                                                                     const uint32_t* __restrict__ src,
                                                                     uint32_t* __restrict__ dst, int64_t words) {
  if (int(blockIdx.x) < upload_blocks) {
    upload_block(src, dst, words, blockIdx.x);
    return;
  }
  merge_blocks<D>(a, int(blockIdx.x) - upload_blocks, int(gridDim.x) - upload_blocks);
}

// Streaming read (a measurement hook, not part of the method): every 16-byte piece of the buffer
// is loaded exactly once, four independent loads per thread in flight, non-temporal (the data is
// not reused).  Each thread stores the XOR of the words it read, so the XOR over all stores is the
// XOR of the buffer's words: the caller can check that every byte was read.
constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                    uint32_t* __restrict__ sink) {
  const int64_t tid = int64_t(blockIdx.x) * kReadThreads + threadIdx.x;
  const int64_t stride = int64_t(gridDim.x) * kReadThreads;
  uint32_t x = 0;
  int64_t i = tid;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[tid] = x;
}

// ---------------------------------------------------------------- host launchers

// Block read (a measurement hook, not part of the method): 4 KB blocks of the buffer visited in a
// given order, the access pattern of paged K/V (a page of one head's 16 keys is 4 KB at d = 128):
// each wave reads whole blocks, two in flight (the decode's K and V of one key block), with 16-byte
// non-temporal loads; block indices past the buffer are clamped to its last block.
constexpr int kBlockWords16 = 4096 / 16;

__global__ __launch_bounds__(kReadThreads) void block_read_kernel(const u32x4* __restrict__ src, int64_t n_buf_blocks,
                                                                   const int32_t* __restrict__ order, int32_t n_blocks,
                                                                   uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = int64_t(blockIdx.x) * (kReadThreads / 64) + (threadIdx.x >> 6);
  const int64_t nw = int64_t(gridDim.x) * (kReadThreads / 64);
  auto base = [&](int64_t b) {
    const int64_t p = min(max(int64_t(order[b]), int64_t(0)), n_buf_blocks - 1);
    return p * kBlockWords16 + lane;
  };
  uint32_t x = 0;
  int64_t b = gw;
  for (; b + nw < n_blocks; b += 2 * nw) {
    const int64_t p0 = base(b), p1 = base(b + nw);
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = __builtin_nontemporal_load(src + p0 + 64 * u);
      v[4 + u] = __builtin_nontemporal_load(src + p1 + 64 * u);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; b < n_blocks; b += nw) {
    const int64_t p0 = base(b);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 v = __builtin_nontemporal_load(src + p0 + 64 * u);
      x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  sink[int64_t(blockIdx.x) * kReadThreads + threadIdx.x] = x;
}

int stream_read_threads() { return kReadThreads; }

hipError_t launch_block_read(const void* src, int64_t n_buf_blocks, const int32_t* order, int32_t n_blocks,
                             uint32_t* sink, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(block_read_kernel, dim3(grid), dim3(kReadThreads), 0, stream, static_cast<const u32x4*>(src),
                     n_buf_blocks, order, n_blocks, sink);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t n16, uint32_t* sink, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kReadThreads), 0, stream, static_cast<const u32x4*>(src),
                     n16, sink);
  return hipGetLastError();
}

hipError_t launch_plan_upload(const void* src_dev, void* dst, int64_t words, hipStream_t stream) {
  const int64_t grid = (words + kUploadWordsPerBlock - 1) / kUploadWordsPerBlock;
  if (grid < 1 || grid > (int64_t(1) << 30)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_upload_kernel, dim3(unsigned(grid)), dim3(256), 0, stream,
                     static_cast<const uint32_t*>(src_dev), static_cast<uint32_t*>(dst), words);
  return hipGetLastError();
}

hipError_t launch_merge(int head_dim, const MergeArgs& a, int grid, hipStream_t stream) {
  if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(kMergeThreads), 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(kMergeThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_merge_upload(int head_dim, const MergeArgs& a, int merge_grid, const void* src_dev, void* dst,
                               int64_t words, hipStream_t stream) {
  const int64_t up = (words + kUploadWordsPerBlock - 1) / kUploadWordsPerBlock;
  if (up < 1 || merge_grid < 1 || up + merge_grid > (int64_t(1) << 30)) return hipErrorInvalidValue;
  const dim3 grid(unsigned(up + merge_grid));
  const uint32_t* s = static_cast<const uint32_t*>(src_dev);
  uint32_t* d = static_cast<uint32_t*>(dst);
  if (head_dim == 128)
    hipLaunchKernelGGL(merge_upload_kernel<128>, grid, dim3(kMergeThreads), 0, stream, a, int(up), s, d, words);
  else if (head_dim == 64)
    hipLaunchKernelGGL(merge_upload_kernel<64>, grid, dim3(kMergeThreads), 0, stream, a, int(up), s, d, words);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_merge_pair(const float* oa, const float* la, const float* ob, const float* lb, void* out,
                             float* lse_out, int rows, int D, int out_bf16, hipStream_t stream) {
  const int64_t total = int64_t(rows) * (D / 4);
  int grid = int((total + kMergeThreads - 1) / kMergeThreads);
  grid = grid < 1 ? 1 : (grid > 4096 ? 4096 : grid);
  hipLaunchKernelGGL(merge_pair_kernel, dim3(grid), dim3(kMergeThreads), 0, stream, oa, la, ob, lb, out, lse_out,
                     rows, D, out_bf16);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* table, int n_pos, int D, double theta, hipStream_t stream) {
  const int64_t total = int64_t(n_pos) * (D / 2);
  int grid = int((total + 255) / 256);
  grid = grid < 1 ? 1 : (grid > 8192 ? 8192 : grid);
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid), dim3(256), 0, stream, table, n_pos, D, theta);
  return hipGetLastError();
}

hipError_t launch_gather(int dtype, int head_dim, bool dense, const AttnArgs& a, const int64_t* row_off, void* k_out,
                         void* v_out, int grid, hipStream_t stream) {
#define BSK_GATHER(T, D, DN)                                                                                     \
  if (head_dim == D && dense == DN) {                                                                            \
    hipLaunchKernelGGL((gather_kernel<T, D, DN>), dim3(grid), dim3(256), 0, stream, a, row_off,                  \
                       static_cast<T*>(k_out), static_cast<T*>(v_out));                                          \
    return hipGetLastError();                                                                                    \
  }
  if (dtype == 1) {
    BSK_GATHER(__bf16, 128, false)
    BSK_GATHER(__bf16, 128, true)
    BSK_GATHER(__bf16, 64, false)
    BSK_GATHER(__bf16, 64, true)
  } else {
    BSK_GATHER(float, 128, false)
    BSK_GATHER(float, 128, true)
    BSK_GATHER(float, 64, false)
    BSK_GATHER(float, 64, true)
  }
#undef BSK_GATHER
  return hipErrorInvalidValue;
}

}  // namespace bsk
