// C ABI of libbsk: argument validation, plan upload and kernel dispatch.
// The entry points and their contracts are declared in include/bsk.h.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <cstring>
#include <string>

#include "../../include/bsk.h"
#include "launch.h"
#include "plan.h"

namespace {

thread_local std::string g_err;

bsk_status fail(bsk_status code, const std::string& msg) {
  g_err = msg;
  return code;
}

bsk_status hip_fail(hipError_t e, const char* what) {
  return fail(BSK_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// The equal-stride kernels are used when the caller allows it and K and V share all strides.
bool same_kv(const bsk_problem& p, const bsk_tensors& t) {
  return p.independent_kv_strides == 0 && t.k_stride_head == t.v_stride_head && t.k_stride_tok == t.v_stride_tok &&
         (p.kv_mode == BSK_KV_DENSE || t.k_stride_page == t.v_stride_page);
}

bool is_prefill_tile(int tile_q) { return tile_q == BSK_TILE_PREFILL || tile_q == BSK_TILE_PREFILL_256; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Largest chunk (keys) whose page ids fit the kernels' LDS page list.
int32_t kernel_chunk_cap(const bsk_problem& p) {
  if (p.kv_mode == BSK_KV_DENSE) return 0;
  const int64_t cap = int64_t(bsk::kMaxPages) * p.page_size;
  return int32_t(std::min<int64_t>(cap / p.tile_kv * p.tile_kv, INT32_MAX / 2));
}

bsk_status check_problem(const bsk_problem* p) {
  if (!p) return fail(BSK_ERR_INVALID_ARG, "problem is NULL");
  if (p->num_qo_heads <= 0 || p->num_kv_heads <= 0 || p->num_qo_heads % p->num_kv_heads != 0)
    return fail(BSK_ERR_INVALID_ARG, "num_qo_heads must be a positive multiple of num_kv_heads");
  if (p->head_dim != 64 && p->head_dim != 128) return fail(BSK_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (p->dtype != BSK_DTYPE_F32 && p->dtype != BSK_DTYPE_BF16) return fail(BSK_ERR_UNSUPPORTED, "dtype");
  if (p->out_dtype != BSK_DTYPE_F32 && p->out_dtype != BSK_DTYPE_BF16) return fail(BSK_ERR_UNSUPPORTED, "out_dtype");
  if (p->kv_mode != BSK_KV_PAGED && p->kv_mode != BSK_KV_DENSE) return fail(BSK_ERR_INVALID_ARG, "kv_mode");
  if (p->kv_mode == BSK_KV_PAGED && (!is_pow2(p->page_size) || p->page_size > 65536))
    return fail(BSK_ERR_INVALID_ARG, "page_size must be a power of two <= 65536");
  if (p->causal != 0 && p->causal != 1) return fail(BSK_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->fused_merge != 0 && p->fused_merge != 1) return fail(BSK_ERR_INVALID_ARG, "fused_merge must be 0 or 1");
  if (p->independent_kv_strides != 0 && p->independent_kv_strides != 1)
    return fail(BSK_ERR_INVALID_ARG, "independent_kv_strides must be 0 or 1");
  if (p->decode_tile_q != 0 && (p->decode_tile_q != BSK_TILE_DECODE || p->tile_q != BSK_TILE_PREFILL))
    return fail(BSK_ERR_INVALID_ARG, "decode_tile_q must be 0, or 16 with tile_q 128");
  if (p->decode_tile_q != 0 && p->kv_mode != BSK_KV_PAGED)
    return fail(BSK_ERR_UNSUPPORTED, "the mixed launch is built for the paged layout only");
  if (p->shared_prefix_len < 0) return fail(BSK_ERR_INVALID_ARG, "shared_prefix_len must be >= 0");
  if (p->shared_prefix_len > 0 &&
      (p->tile_q != BSK_TILE_PREFILL || p->decode_tile_q != BSK_TILE_DECODE || p->kv_mode != BSK_KV_PAGED))
    return fail(BSK_ERR_INVALID_ARG, "a shared prefix needs tile_q 128, decode_tile_q 16 and paged suffixes");
  if (p->shared_prefix_len > 0 && (p->window > 0 || p->rope_mode != BSK_ROPE_NONE || p->fused_merge != 0))
    return fail(BSK_ERR_UNSUPPORTED, "a shared prefix is built without window, RoPE and in-kernel merge");
  if (p->window > 0 && p->sink < 0) return fail(BSK_ERR_INVALID_ARG, "sink must be >= 0");
  if (p->rope_mode < BSK_ROPE_NONE || p->rope_mode > BSK_ROPE_ABSOLUTE) return fail(BSK_ERR_INVALID_ARG, "rope_mode");
  if (p->rope_mode == BSK_ROPE_STREAMING && !p->causal)
    return fail(BSK_ERR_INVALID_ARG, "streaming RoPE positions need causal masking");
  if (p->rope_mode != BSK_ROPE_NONE && !(p->rope_theta > 1.0)) return fail(BSK_ERR_INVALID_ARG, "rope_theta must be > 1");
  if (!std::isfinite(p->sm_scale) || !(p->sm_scale > 0.f)) return fail(BSK_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  if (p->tile_q != BSK_TILE_DECODE && !is_prefill_tile(p->tile_q))
    return fail(BSK_ERR_INVALID_ARG, "tile_q must be 16 (decode) or 128 / 256 (prefill)");
  if (p->tile_kv <= 0 || (p->kv_mode == BSK_KV_PAGED && p->tile_kv % p->page_size != 0))
    return fail(BSK_ERR_INVALID_ARG, "tile_kv must be a positive multiple of page_size");
  if (p->num_workers <= 0 || p->split_factor <= 0) return fail(BSK_ERR_INVALID_ARG, "num_workers, split_factor");
  if (p->min_chunk <= 0 || p->min_chunk % p->tile_kv) return fail(BSK_ERR_INVALID_ARG, "min_chunk");
  if (p->max_batch < 0 || p->max_items_per_worker <= 0 || p->max_slots < 0 || p->max_merge < 0)
    return fail(BSK_ERR_INVALID_ARG, "capacities");
  const int32_t cap = kernel_chunk_cap(*p);
  if (cap > 0) {
    if (p->max_chunk > cap) return fail(BSK_ERR_INVALID_ARG, "max_chunk exceeds the kernels' page-list capacity");
    if (p->min_chunk > cap) return fail(BSK_ERR_INVALID_ARG, "min_chunk exceeds the kernels' page-list capacity");
    if (p->window > 0 && int64_t(p->sink) > int64_t(bsk::kMaxPages) * p->page_size)
      return fail(BSK_ERR_INVALID_ARG, "sink range exceeds the kernels' page-list capacity");
  }
  return BSK_OK;
}

bsk::PlanParams plan_params(const bsk_problem& p) {
  bsk::PlanParams q;
  q.num_qo_heads = p.num_qo_heads;
  q.num_kv_heads = p.num_kv_heads;
  q.tile_q = p.tile_q;
  q.tile_kv = p.tile_kv;
  q.num_workers = p.num_workers;
  q.split_factor = p.split_factor;
  q.min_chunk = p.min_chunk;
  q.max_chunk = p.max_chunk > 0 ? p.max_chunk : kernel_chunk_cap(p);
  q.item_overhead = p.item_overhead;
  q.max_batch = p.max_batch;
  q.max_items_per_worker = p.max_items_per_worker;
  q.max_slots = p.max_slots;
  q.max_merge = p.max_merge;
  q.causal = p.causal != 0;
  q.window = p.window > 0 ? p.window : 0;
  q.sink = p.window > 0 ? p.sink : 0;
  q.decode_tile_q = p.decode_tile_q;
  q.shared_prefix_len = p.shared_prefix_len;
  return q;
}

size_t float_ws_need(const bsk_problem& p) {
  return size_t(p.max_slots) * size_t(p.tile_q) * size_t(p.head_dim + 1) * sizeof(float);
}

// The plan must have been built for this problem: the kernels take the slot stride and the launch
// grid from the problem, the item and merge records from the plan.
bsk_status check_plan_matches(const bsk_problem& p, const bsk_plan_info& info) {
  if (info.tile_q != p.tile_q) return fail(BSK_ERR_INVALID_ARG, "plan was built for another query-tile class");
  if (info.num_workers != p.num_workers) return fail(BSK_ERR_INVALID_ARG, "plan info does not match problem");
  if (info.num_slots < 0 || info.num_slots > p.max_slots || info.num_merge < 0 || info.num_merge > p.max_merge)
    return fail(BSK_ERR_INVALID_ARG, "plan slots / merge entries exceed the problem's capacities");
  return BSK_OK;
}

// Everything a run checks except the float workspace.
bsk_status check_run_inputs(const bsk_problem* p, const bsk_plan_info* info, const bsk_tensors* t,
                            const void* int_ws, int tile_q) {
  bsk_status s = check_problem(p);
  if (s != BSK_OK) return s;
  if (!info || !t || !int_ws) return fail(BSK_ERR_INVALID_ARG, "plan info, tensors and int workspace are required");
  const bool want_prefill = tile_q != BSK_TILE_DECODE;
  if (want_prefill ? !is_prefill_tile(p->tile_q) : p->tile_q != tile_q)
    return fail(BSK_ERR_INVALID_ARG, "plan was built for the other query-tile class");
  s = check_plan_matches(*p, *info);
  if (s != BSK_OK) return s;
  const size_t ebytes = p->dtype == BSK_DTYPE_BF16 ? 2 : 4;
  const int64_t vec = 16 / int64_t(ebytes);
  if (!t->q || !t->k || !t->v || !t->out || !t->lse) return fail(BSK_ERR_INVALID_ARG, "null tensor");
  if (!aligned(t->q, 16) || !aligned(t->k, 16) || !aligned(t->v, 16))
    return fail(BSK_ERR_INVALID_ARG, "q, k, v must be 16-byte aligned");
  if (t->q_stride_tok % vec || t->q_stride_head % vec || t->k_stride_head % vec || t->k_stride_tok % vec ||
      t->v_stride_head % vec || t->v_stride_tok % vec ||
      (p->kv_mode == BSK_KV_PAGED && (t->k_stride_page % vec || t->v_stride_page % vec)))
    return fail(BSK_ERR_INVALID_ARG, "q/k/v strides must be multiples of 16 bytes");
  if (!aligned(t->out, p->out_dtype == BSK_DTYPE_F32 ? 16 : 8) || t->o_stride_tok % 4 || t->o_stride_head % 4)
    return fail(BSK_ERR_INVALID_ARG, "out must be aligned to 4 elements (strides too)");
  if (p->kv_mode == BSK_KV_PAGED && !t->kv_page_indices) return fail(BSK_ERR_INVALID_ARG, "kv_page_indices is NULL");
  if (p->shared_prefix_len > 0) {
    if (!t->prefix_k || !t->prefix_v || !aligned(t->prefix_k, 16) || !aligned(t->prefix_v, 16))
      return fail(BSK_ERR_INVALID_ARG, "prefix_k / prefix_v missing or not 16-byte aligned");
    if (t->prefix_k_stride_tok % vec || t->prefix_k_stride_head % vec || t->prefix_v_stride_tok % vec ||
        t->prefix_v_stride_head % vec)
      return fail(BSK_ERR_INVALID_ARG, "prefix strides must be multiples of 16 bytes");
  }
  if (p->rope_mode != BSK_ROPE_NONE) {
    if (!t->rope_cos_sin || !aligned(t->rope_cos_sin, 16)) return fail(BSK_ERR_INVALID_ARG, "rope table missing");
    int64_t need = info->max_kv_len;
    if (p->rope_mode == BSK_ROPE_STREAMING && p->window > 0)
      need = std::min<int64_t>(need, int64_t(p->window) + p->sink);
    if (t->rope_n_pos < need) return fail(BSK_ERR_INVALID_ARG, "rope table has too few positions");
    if (p->rope_mode == BSK_ROPE_STREAMING && info->max_qo_len > 1)
      return fail(BSK_ERR_UNSUPPORTED, "streaming RoPE positions are per query; needs qo_len <= 1");
  }
  return BSK_OK;
}

bsk_status check_run(const bsk_problem* p, const bsk_plan_info* info, const bsk_tensors* t, const void* int_ws,
                     void* float_ws, size_t float_ws_bytes, int tile_q) {
  bsk_status s = check_run_inputs(p, info, t, int_ws, tile_q);
  if (s != BSK_OK) return s;
  if (info->num_slots > 0 && (!float_ws || float_ws_bytes < float_ws_need(*p)))
    return fail(BSK_ERR_WORKSPACE, "float workspace smaller than bsk_workspace_query");
  return BSK_OK;
}

bsk::AttnArgs attn_args(const bsk_problem& p, const bsk_tensors& t, const void* int_ws, float* part_o,
                        float* part_lse) {
  bsk::AttnArgs a;
  a.q = t.q;
  a.q_st = t.q_stride_tok;
  a.q_sh = t.q_stride_head;
  a.k = t.k;
  a.v = t.v;
  a.k_sp = t.k_stride_page;
  a.k_sh = t.k_stride_head;
  a.k_st = t.k_stride_tok;
  a.v_sp = t.v_stride_page;
  a.v_sh = t.v_stride_head;
  a.v_st = t.v_stride_tok;
  a.page_indices = t.kv_page_indices;
  a.out = t.out;
  a.o_st = t.o_stride_tok;
  a.o_sh = t.o_stride_head;
  a.lse = t.lse;
  a.lse_st = t.lse_stride_tok;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.ws = static_cast<const int32_t*>(int_ws);
  a.ws_rw = static_cast<int32_t*>(const_cast<void*>(int_ws));
  a.fused_merge = p.fused_merge != 0;
  a.rope = t.rope_cos_sin;
  a.rope_n_pos = t.rope_n_pos;
  a.pk = p.shared_prefix_len > 0 ? t.prefix_k : nullptr;
  a.pv = p.shared_prefix_len > 0 ? t.prefix_v : nullptr;
  a.pk_st = t.prefix_k_stride_tok;
  a.pk_sh = t.prefix_k_stride_head;
  a.pv_st = t.prefix_v_stride_tok;
  a.pv_sh = t.prefix_v_stride_head;
  a.group = p.num_qo_heads / p.num_kv_heads;
  a.page_shift = p.kv_mode == BSK_KV_PAGED ? ilog2(p.page_size) : 0;
  a.causal = p.causal;
  a.window = p.window > 0 ? p.window : 0;
  a.sink = p.window > 0 ? p.sink : 0;
  a.out_bf16 = p.out_dtype == BSK_DTYPE_BF16;
  a.scale_log2 = float(double(p.sm_scale) * 1.4426950408889634);
  return a;
}

// Partial states in a caller's float workspace: [max_slots][tile_q][D] outputs, then
// [max_slots][tile_q] LSEs.
bsk::AttnArgs attn_args(const bsk_problem& p, const bsk_tensors& t, const void* int_ws, void* float_ws) {
  float* fw = static_cast<float*>(float_ws);
  return attn_args(p, t, int_ws, fw, fw ? fw + size_t(p.max_slots) * p.tile_q * p.head_dim : nullptr);
}

bsk::MergeArgs merge_args(const bsk_problem& p, const bsk_tensors& t, const void* int_ws, const float* part_o,
                          const float* part_lse) {
  bsk::MergeArgs a;
  a.ws = static_cast<const int32_t*>(int_ws);
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.out = t.out;
  a.o_st = t.o_stride_tok;
  a.o_sh = t.o_stride_head;
  a.lse = t.lse;
  a.lse_st = t.lse_stride_tok;
  a.group = p.num_qo_heads / p.num_kv_heads;
  a.out_bf16 = p.out_dtype == BSK_DTYPE_BF16;
  return a;
}

// Fixed merge grid: enough blocks for every (entry, row) pair of a full merge table, capped at four
// per compute unit (the blocks loop; idle blocks only cost their dispatch).
int merge_grid(const bsk_problem& p) {
  const int64_t rows_per_block = 256 / (p.head_dim / 4);
  const int64_t want = (int64_t(p.max_merge) * p.tile_q + rows_per_block - 1) / rows_per_block;
  return int(want < 1 ? 1 : (want > 1024 ? 1024 : want));
}

bsk_status launch_run(const bsk_problem& p, const bsk_plan_info& info, const bsk_tensors& t, const bsk::AttnArgs& a,
                      hipStream_t stream) {
  hipError_t e;
  if (p.tile_q == BSK_TILE_DECODE)
    e = bsk::launch_decode(p.dtype, p.head_dim, p.kv_mode == BSK_KV_DENSE, p.rope_mode, same_kv(p, t), a,
                           info.num_workers, stream);
  else if (p.decode_tile_q != 0)
    e = bsk::launch_mixed(p.head_dim, same_kv(p, t), a, info.num_workers, stream);
  else
    e = bsk::launch_prefill(p.head_dim, p.kv_mode == BSK_KV_DENSE, p.tile_q, same_kv(p, t), a, info.num_workers,
                            stream);
  if (e != hipSuccess) return hip_fail(e, p.tile_q == BSK_TILE_DECODE ? "decode launch" : "prefill launch");
  return BSK_OK;
}

// Checks of the decode-class run beyond check_run_inputs.
bsk_status check_decode(const bsk_problem* problem) {
  if (problem->rope_mode != BSK_ROPE_NONE && problem->dtype != BSK_DTYPE_BF16)
    return fail(BSK_ERR_UNSUPPORTED, "fused RoPE is built for bf16 only");
  if (problem->rope_mode != BSK_ROPE_NONE && problem->kv_mode != BSK_KV_PAGED)
    return fail(BSK_ERR_UNSUPPORTED, "fused RoPE is built for the paged layout only");
  return BSK_OK;
}

// Checks of the prefill-class run beyond check_run_inputs.
bsk_status check_prefill(const bsk_problem* problem, const bsk_tensors* t) {
  if (problem->dtype != BSK_DTYPE_BF16) return fail(BSK_ERR_UNSUPPORTED, "the prefill kernel is bf16 only");
  if (problem->rope_mode != BSK_ROPE_NONE) return fail(BSK_ERR_UNSUPPORTED, "fused RoPE is built for decode only");
  // the kernel forms page addresses with a 32 x 32 -> 64-bit multiply of the page id and the byte stride
  // and keeps a row's head / in-page (dense: in-tile) offset in 32 bits
  if (problem->kv_mode == BSK_KV_PAGED &&
      (t->k_stride_page < 0 || t->v_stride_page < 0 || t->k_stride_page > INT32_MAX || t->v_stride_page > INT32_MAX))
    return fail(BSK_ERR_INVALID_ARG, "page strides must be in [0, 2^31) elements");
  const int64_t rows = problem->kv_mode == BSK_KV_PAGED ? std::min(problem->page_size, 64) : 64;
  const int64_t hk = problem->num_kv_heads;
  const int64_t kspan = (hk - 1) * t->k_stride_head + (rows - 1) * t->k_stride_tok + problem->head_dim;
  const int64_t vspan = (hk - 1) * t->v_stride_head + (rows - 1) * t->v_stride_tok + problem->head_dim;
  if (t->k_stride_head < 0 || t->k_stride_tok < 0 || t->v_stride_head < 0 || t->v_stride_tok < 0 ||
      kspan > INT32_MAX || vspan > INT32_MAX)
    return fail(BSK_ERR_INVALID_ARG, "head / token strides too large for the prefill kernel's 32-bit row offsets");
  if (problem->shared_prefix_len > 0) {
    // the dense prefix tiles are 64 rows of consecutive tokens
    const int64_t pks = (hk - 1) * t->prefix_k_stride_head + 63 * t->prefix_k_stride_tok + problem->head_dim;
    const int64_t pvs = (hk - 1) * t->prefix_v_stride_head + 63 * t->prefix_v_stride_tok + problem->head_dim;
    if (t->prefix_k_stride_tok < 0 || t->prefix_k_stride_head < 0 || t->prefix_v_stride_tok < 0 ||
        t->prefix_v_stride_head < 0 || pks > INT32_MAX || pvs > INT32_MAX)
      return fail(BSK_ERR_INVALID_ARG, "prefix strides too large for the prefill kernel's 32-bit row offsets");
  }
  return BSK_OK;
}

// Copies the plan's first `used_bytes` from host_ws into the int workspace on `stream`.  Pinned
// host memory has a device address: a kernel copies the plan from there (one launch, ordered with
// the caller's kernels).  Other host memory goes through hipMemcpyAsync.
bsk_status upload_plan(const void* host_ws, void* int_ws_dev, int64_t used_bytes, hipStream_t stream) {
  void* src_dev = nullptr;
  hipError_t e = hipHostGetDevicePointer(&src_dev, const_cast<void*>(host_ws), 0);
  if (e == hipSuccess && src_dev && aligned(src_dev, 16) && aligned(int_ws_dev, 16)) {
    e = bsk::launch_plan_upload(src_dev, int_ws_dev, used_bytes / int64_t(sizeof(int32_t)), stream);
    if (e != hipSuccess) return hip_fail(e, "plan upload kernel");
  } else {
    if (e != hipSuccess) (void)hipGetLastError();  // not pinned host memory: not an error here
    e = hipMemcpyAsync(int_ws_dev, host_ws, size_t(used_bytes), hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(plan)");
  }
  return BSK_OK;
}

// The arguments of a deferred upload of a plan built by bsk_plan for `problem`.
bsk_status check_upload(const bsk_problem* problem, const bsk_plan_info* info, const void* host_ws,
                        size_t host_ws_bytes, const void* int_ws_dev, size_t int_ws_bytes) {
  bsk_status s = check_problem(problem);
  if (s != BSK_OK) return s;
  if (!info || !host_ws || !int_ws_dev) return fail(BSK_ERR_INVALID_ARG, "plan info, host and int workspaces are required");
  s = check_plan_matches(*problem, *info);
  if (s != BSK_OK) return s;
  if (int_ws_bytes < bsk::plan_workspace_bytes(plan_params(*problem)))
    return fail(BSK_ERR_WORKSPACE, "int workspace smaller than bsk_workspace_query");
  if (info->used_bytes <= 0 || info->used_bytes % int64_t(sizeof(int32_t)) != 0 ||
      uint64_t(info->used_bytes) > host_ws_bytes || uint64_t(info->used_bytes) > int_ws_bytes)
    return fail(BSK_ERR_INVALID_ARG, "plan size does not fit the host or int workspace");
  return BSK_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

const char* bsk_status_string(bsk_status status) {
  switch (status) {
    case BSK_OK: return "BSK_OK";
    case BSK_ERR_INVALID_ARG: return "BSK_ERR_INVALID_ARG";
    case BSK_ERR_UNSUPPORTED: return "BSK_ERR_UNSUPPORTED";
    case BSK_ERR_CAPACITY: return "BSK_ERR_CAPACITY";
    case BSK_ERR_WORKSPACE: return "BSK_ERR_WORKSPACE";
    case BSK_ERR_HIP: return "BSK_ERR_HIP";
    default: return "BSK_ERR_UNKNOWN";
  }
}

const char* bsk_last_error(void) { return g_err.c_str(); }

bsk_status bsk_device_workers(const bsk_problem* problem, int32_t* num_workers) {
  if (!num_workers) return fail(BSK_ERR_INVALID_ARG, "num_workers is NULL");
  if (!problem) return fail(BSK_ERR_INVALID_ARG, "problem is NULL");
  if (problem->head_dim != 64 && problem->head_dim != 128) return fail(BSK_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const bool dense = problem->kv_mode == BSK_KV_DENSE;
  const void* fn = nullptr;
  int threads = 0;
  if (problem->tile_q == BSK_TILE_DECODE) {
    fn = bsk::decode_kernel_ptr(problem->dtype, problem->head_dim, dense, problem->rope_mode,
                                problem->independent_kv_strides == 0);
    threads = bsk::decode_threads();
  } else if (is_prefill_tile(problem->tile_q)) {
    if (problem->dtype == BSK_DTYPE_BF16 && problem->rope_mode == BSK_ROPE_NONE)
      fn = problem->decode_tile_q != 0
               ? bsk::mixed_kernel_ptr(problem->head_dim, problem->independent_kv_strides == 0)
               : bsk::prefill_kernel_ptr(problem->head_dim, dense, problem->tile_q,
                                         problem->independent_kv_strides == 0);
    threads = problem->decode_tile_q != 0 ? bsk::prefill_threads(128) : bsk::prefill_threads(problem->tile_q);
  } else {
    return fail(BSK_ERR_INVALID_ARG, "tile_q must be 16, 128 or 256");
  }
  if (!fn) return fail(BSK_ERR_UNSUPPORTED, "no kernel built for this dtype / layout / RoPE combination");
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0);
  if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  int per = per_cu > 0 ? per_cu : 1;
  // The decode kernels fit three workgroups per CU but are planned over two: fewer, longer items
  // measured 1-2 us faster per step from batch 32 up (Llama-3 lengths) and 0.3 us slower at 16.
  if (problem->tile_q == BSK_TILE_DECODE) per = std::min(per, 2);
  *num_workers = cus * per;
  return BSK_OK;
}

bsk_status bsk_workspace_query(const bsk_problem* problem, size_t* int_ws_bytes, size_t* float_ws_bytes,
                               size_t* host_ws_bytes) {
  bsk_status s = check_problem(problem);
  if (s != BSK_OK) return s;
  const size_t ib = bsk::plan_workspace_bytes(plan_params(*problem));
  if (int_ws_bytes) *int_ws_bytes = ib;
  if (host_ws_bytes) *host_ws_bytes = ib;
  if (float_ws_bytes) *float_ws_bytes = float_ws_need(*problem);
  return BSK_OK;
}

bsk_status bsk_plan(const bsk_problem* problem, int32_t batch, const int32_t* qo_indptr, const int32_t* kv_len,
                    const int32_t* kv_indptr, void* host_ws, size_t host_ws_bytes, void* int_ws_dev,
                    size_t int_ws_bytes, void* stream, bsk_plan_info* info) {
  bsk_status s = check_problem(problem);
  if (s != BSK_OK) return s;
  if (!info) return fail(BSK_ERR_INVALID_ARG, "info is NULL");
  const bsk::PlanParams pp = plan_params(*problem);
  if (problem->kv_mode == BSK_KV_PAGED && batch > 0 && kv_indptr && kv_len) {
    for (int32_t r = 0; r < batch; ++r) {
      const int64_t pages = int64_t(kv_indptr[r + 1]) - kv_indptr[r];
      if (pages < 0 || int64_t(kv_len[r]) > pages * problem->page_size)
        return fail(BSK_ERR_INVALID_ARG, "request " + std::to_string(r) + " has fewer pages than kv_len needs");
    }
  }
  if (int_ws_dev && int_ws_bytes < bsk::plan_workspace_bytes(pp))
    return fail(BSK_ERR_WORKSPACE, "int workspace smaller than bsk_workspace_query");
  bsk::PlanStats st;
  std::string err;
  const bsk::PlanResult pr = bsk::build_plan(pp, batch, qo_indptr, kv_len, kv_indptr, static_cast<int32_t*>(host_ws),
                                             host_ws_bytes, &st, &err);
  if (pr == bsk::PLAN_CAPACITY) return fail(BSK_ERR_CAPACITY, err);
  if (pr == bsk::PLAN_WORKSPACE) return fail(BSK_ERR_WORKSPACE, err);
  if (pr != bsk::PLAN_OK) return fail(BSK_ERR_INVALID_ARG, err);
  std::memset(info, 0, sizeof(*info));
  info->num_workers = problem->num_workers;
  info->tile_q = problem->tile_q;
  info->batch = batch;
  info->num_items = st.num_items;
  info->num_slots = st.num_slots;
  info->num_merge = st.num_merge;
  info->chunk = st.chunk;
  info->max_kv_len = st.max_kv_len;
  info->max_qo_len = st.max_qo_len;
  info->max_items_on_worker = st.max_items_on_worker;
  info->total_cost = st.total_cost;
  info->max_load = st.max_load;
  info->used_bytes = st.used_bytes;
  if (int_ws_dev) return upload_plan(host_ws, int_ws_dev, st.used_bytes, static_cast<hipStream_t>(stream));
  return BSK_OK;
}

bsk_status bsk_upload_plan(const bsk_problem* problem, const bsk_plan_info* info, const void* host_ws,
                           size_t host_ws_bytes, void* int_ws_dev, size_t int_ws_bytes, void* stream) {
  bsk_status s = check_upload(problem, info, host_ws, host_ws_bytes, int_ws_dev, int_ws_bytes);
  if (s != BSK_OK) return s;
  return upload_plan(host_ws, int_ws_dev, info->used_bytes, static_cast<hipStream_t>(stream));
}

bsk_status bsk_run_decode(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                          void* int_ws_dev, void* float_ws, size_t float_ws_bytes, void* stream) {
  bsk_status s = check_run(problem, info, t, int_ws_dev, float_ws, float_ws_bytes, BSK_TILE_DECODE);
  if (s == BSK_OK) s = check_decode(problem);
  if (s != BSK_OK) return s;
  return launch_run(*problem, *info, *t, attn_args(*problem, *t, int_ws_dev, float_ws),
                    static_cast<hipStream_t>(stream));
}

bsk_status bsk_run_prefill(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                           void* int_ws_dev, void* float_ws, size_t float_ws_bytes, void* stream) {
  bsk_status s = check_run(problem, info, t, int_ws_dev, float_ws, float_ws_bytes, BSK_TILE_PREFILL);
  if (s == BSK_OK) s = check_prefill(problem, t);
  if (s != BSK_OK) return s;
  return launch_run(*problem, *info, *t, attn_args(*problem, *t, int_ws_dev, float_ws),
                    static_cast<hipStream_t>(stream));
}

bsk_status bsk_merge_states(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                            const void* int_ws_dev, const void* float_ws, size_t float_ws_bytes, void* stream) {
  bsk_status s = check_problem(problem);
  if (s != BSK_OK) return s;
  if (!info || !t || !int_ws_dev || !t->out || !t->lse) return fail(BSK_ERR_INVALID_ARG, "null argument");
  s = check_plan_matches(*problem, *info);
  if (s != BSK_OK) return s;
  if (info->num_slots > 0 && (!float_ws || float_ws_bytes < float_ws_need(*problem)))
    return fail(BSK_ERR_WORKSPACE, "float workspace missing or smaller than bsk_workspace_query");
  if (!aligned(t->out, problem->out_dtype == BSK_DTYPE_F32 ? 16 : 8) || t->o_stride_tok % 4 || t->o_stride_head % 4)
    return fail(BSK_ERR_INVALID_ARG, "out must be aligned to 4 elements (strides too)");
  const float* fw = static_cast<const float*>(float_ws);
  const bsk::MergeArgs a =
      merge_args(*problem, *t, int_ws_dev, fw, fw ? fw + size_t(problem->max_slots) * problem->tile_q * problem->head_dim
                                                  : nullptr);
  hipError_t e = bsk::launch_merge(problem->head_dim, a, merge_grid(*problem), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return BSK_OK;
}

bsk_status bsk_merge_states_upload(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                                   const void* int_ws_dev, const void* float_ws, size_t float_ws_bytes,
                                   const bsk_problem* next_problem, const bsk_plan_info* next_info,
                                   const void* next_host_ws, size_t next_host_ws_bytes, void* next_int_ws_dev,
                                   size_t next_int_ws_bytes, void* stream) {
  bsk_status s = check_upload(next_problem, next_info, next_host_ws, next_host_ws_bytes, next_int_ws_dev,
                              next_int_ws_bytes);
  if (s != BSK_OK) return s;
  s = check_problem(problem);
  if (s != BSK_OK) return s;
  if (!info || !t || !int_ws_dev || !t->out || !t->lse) return fail(BSK_ERR_INVALID_ARG, "null argument");
  s = check_plan_matches(*problem, *info);
  if (s != BSK_OK) return s;
  // the merge reads its plan's first used_bytes while the upload writes the next plan's
  if (info->used_bytes <= 0) return fail(BSK_ERR_INVALID_ARG, "plan info holds no plan");
  const uintptr_t a0 = uintptr_t(int_ws_dev), a1 = a0 + uint64_t(info->used_bytes);
  const uintptr_t b0 = uintptr_t(next_int_ws_dev), b1 = b0 + uint64_t(next_info->used_bytes);
  if (a0 < b1 && b0 < a1)
    return fail(BSK_ERR_INVALID_ARG, "the next plan must go to another int workspace than the merged run's");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (info->num_slots > 0 && (!float_ws || float_ws_bytes < float_ws_need(*problem)))
    return fail(BSK_ERR_WORKSPACE, "float workspace missing or smaller than bsk_workspace_query");
  if (!aligned(t->out, problem->out_dtype == BSK_DTYPE_F32 ? 16 : 8) || t->o_stride_tok % 4 || t->o_stride_head % 4)
    return fail(BSK_ERR_INVALID_ARG, "out must be aligned to 4 elements (strides too)");
  const float* fw = static_cast<const float*>(float_ws);
  const bsk::MergeArgs a =
      merge_args(*problem, *t, int_ws_dev, fw, fw ? fw + size_t(problem->max_slots) * problem->tile_q * problem->head_dim
                                                  : nullptr);
  void* src_dev = nullptr;
  hipError_t e = hipHostGetDevicePointer(&src_dev, const_cast<void*>(next_host_ws), 0);
  if (e == hipSuccess && src_dev && aligned(src_dev, 16) && aligned(next_int_ws_dev, 16)) {
    e = bsk::launch_merge_upload(problem->head_dim, a, merge_grid(*problem), src_dev, next_int_ws_dev,
                                 next_info->used_bytes / int64_t(sizeof(int32_t)), st);
    if (e != hipSuccess) return hip_fail(e, "merge + upload launch");
    return BSK_OK;
  }
  if (e != hipSuccess) (void)hipGetLastError();  // not pinned host memory: two steps
  e = bsk::launch_merge(problem->head_dim, a, merge_grid(*problem), st);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return upload_plan(next_host_ws, next_int_ws_dev, next_info->used_bytes, st);
}

bsk_status bsk_run_noalloc(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                           void* int_ws_dev, void* stream) {
  bsk_status s = check_run_inputs(problem, info, t, int_ws_dev, problem ? problem->tile_q : 0);
  if (s == BSK_OK) s = problem->tile_q == BSK_TILE_DECODE ? check_decode(problem) : check_prefill(problem, t);
  if (s != BSK_OK) return s;
  void* base = nullptr;
  size_t bytes = 0;
  hipError_t e = bsk::noalloc_scratch(&base, &bytes);
  if (e != hipSuccess) return hip_fail(e, "scratch address lookup");
  // fixed layout per problem shape: [cap][tile_q][D] partial outputs, then [cap][tile_q] LSEs
  const size_t slot_bytes = size_t(problem->tile_q) * size_t(problem->head_dim + 1) * sizeof(float);
  const int64_t cap = int64_t(bytes / slot_bytes);
  if (info->num_slots > cap)
    return fail(BSK_ERR_CAPACITY, "plan has " + std::to_string(info->num_slots) + " partial-state slots; the " +
                                      std::to_string(bytes >> 20) + " MiB scratch holds " + std::to_string(cap) +
                                      " for this tile_q / head_dim (use bsk_run_* with a float workspace)");
  float* part_o = static_cast<float*>(base);
  float* part_lse = part_o + size_t(cap) * problem->tile_q * problem->head_dim;
  s = launch_run(*problem, *info, *t, attn_args(*problem, *t, int_ws_dev, part_o, part_lse),
                 static_cast<hipStream_t>(stream));
  if (s != BSK_OK || problem->fused_merge) return s;
  e = bsk::launch_merge(problem->head_dim, merge_args(*problem, *t, int_ws_dev, part_o, part_lse),
                        merge_grid(*problem), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return BSK_OK;
}

bsk_status bsk_merge_state_pair(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                                void* o_out, float* lse_out, int32_t rows, int32_t head_dim, int32_t out_dtype,
                                void* stream) {
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return fail(BSK_ERR_INVALID_ARG, "null argument");
  if (rows < 0 || head_dim <= 0 || head_dim % 4) return fail(BSK_ERR_INVALID_ARG, "rows / head_dim");
  if (out_dtype != BSK_DTYPE_F32 && out_dtype != BSK_DTYPE_BF16) return fail(BSK_ERR_INVALID_ARG, "out_dtype");
  if (!aligned(o_a, 16) || !aligned(o_b, 16) || !aligned(o_out, out_dtype == BSK_DTYPE_F32 ? 16 : 8))
    return fail(BSK_ERR_INVALID_ARG, "misaligned state arrays");
  if (rows == 0) return BSK_OK;
  hipError_t e = bsk::launch_merge_pair(o_a, lse_a, o_b, lse_b, o_out, lse_out, rows, head_dim,
                                        out_dtype == BSK_DTYPE_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge pair launch");
  return BSK_OK;
}

bsk_status bsk_rope_table(float* table_dev, int32_t n_pos, int32_t head_dim, double theta, void* stream) {
  if (!table_dev || n_pos <= 0 || head_dim <= 0 || head_dim % 2 || !(theta > 1.0))
    return fail(BSK_ERR_INVALID_ARG, "rope table arguments");
  hipError_t e = bsk::launch_rope_table(table_dev, n_pos, head_dim, theta, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  return BSK_OK;
}

bsk_status bsk_append_paged_kv(const bsk_problem* problem, int32_t batch, int32_t n_total,
                               const int32_t* append_indptr, const int32_t* kv_len, const int32_t* kv_page_indptr,
                               const int32_t* kv_page_indices, const void* k_new, const void* v_new,
                               int64_t new_stride_tok, int64_t new_stride_head, void* k_cache, void* v_cache,
                               int64_t k_stride_page, int64_t k_stride_head, int64_t k_stride_tok,
                               int64_t v_stride_page, int64_t v_stride_head, int64_t v_stride_tok, void* stream) {
  bsk_status s = check_problem(problem);
  if (s != BSK_OK) return s;
  if (problem->kv_mode != BSK_KV_PAGED) return fail(BSK_ERR_INVALID_ARG, "append needs the paged layout");
  if (batch < 0 || n_total < 0) return fail(BSK_ERR_INVALID_ARG, "negative batch / token count");
  if (n_total == 0 || batch == 0) return BSK_OK;
  if (!append_indptr || !kv_len || !kv_page_indptr || !kv_page_indices || !k_new || !v_new || !k_cache || !v_cache)
    return fail(BSK_ERR_INVALID_ARG, "null argument");
  const int64_t vec = 16 / (problem->dtype == BSK_DTYPE_BF16 ? 2 : 4);
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(BSK_ERR_INVALID_ARG, "k_new, v_new and the pools must be 16-byte aligned");
  if (new_stride_tok % vec || new_stride_head % vec || k_stride_page % vec || k_stride_head % vec ||
      k_stride_tok % vec || v_stride_page % vec || v_stride_head % vec || v_stride_tok % vec)
    return fail(BSK_ERR_INVALID_ARG, "strides must be multiples of 16 bytes");
  if (new_stride_tok < 0 || new_stride_head < 0 || k_stride_page < 0 || k_stride_head < 0 || k_stride_tok < 0 ||
      v_stride_page < 0 || v_stride_head < 0 || v_stride_tok < 0)
    return fail(BSK_ERR_INVALID_ARG, "negative strides");
  bsk::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_st = new_stride_tok;
  a.new_sh = new_stride_head;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_sp = k_stride_page;
  a.k_sh = k_stride_head;
  a.k_st = k_stride_tok;
  a.v_sp = v_stride_page;
  a.v_sh = v_stride_head;
  a.v_st = v_stride_tok;
  a.append_indptr = append_indptr;
  a.kv_len = kv_len;
  a.page_indptr = kv_page_indptr;
  a.page_indices = kv_page_indices;
  a.batch = batch;
  a.n_total = n_total;
  a.num_kv_heads = problem->num_kv_heads;
  a.page_shift = ilog2(problem->page_size);
  hipError_t e = bsk::launch_append(problem->dtype, problem->head_dim, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return BSK_OK;
}

bsk_status bsk_rope_apply(const bsk_problem* problem, int32_t batch, int32_t max_kv_len, const int32_t* qo_indptr,
                          const int32_t* kv_len, const int32_t* kv_page_indptr, const bsk_tensors* t, void* q_out,
                          int64_t qo_stride_tok, int64_t qo_stride_head, void* k_out, void* stream) {
  bsk_status s = check_problem(problem);
  if (s != BSK_OK) return s;
  if (problem->dtype != BSK_DTYPE_BF16) return fail(BSK_ERR_UNSUPPORTED, "the unfused RoPE pass is bf16 only");
  if (problem->kv_mode != BSK_KV_PAGED) return fail(BSK_ERR_UNSUPPORTED, "the unfused RoPE pass needs paged KV");
  if (problem->rope_mode == BSK_ROPE_NONE) return fail(BSK_ERR_INVALID_ARG, "rope_mode is NONE");
  if (batch < 0 || max_kv_len < 0) return fail(BSK_ERR_INVALID_ARG, "negative batch / max_kv_len");
  if (batch == 0) return BSK_OK;
  if (!t || !qo_indptr || !kv_len || !kv_page_indptr || !t->q || !t->k || !t->kv_page_indices || !t->rope_cos_sin ||
      !q_out || !k_out)
    return fail(BSK_ERR_INVALID_ARG, "null argument");
  if (!aligned(t->q, 16) || !aligned(t->k, 16) || !aligned(q_out, 16) || !aligned(k_out, 16) ||
      !aligned(t->rope_cos_sin, 16))
    return fail(BSK_ERR_INVALID_ARG, "q, k, q_out, k_out and the table must be 16-byte aligned");
  if (t->q_stride_tok % 8 || t->q_stride_head % 8 || qo_stride_tok % 8 || qo_stride_head % 8 ||
      t->k_stride_page % 8 || t->k_stride_head % 8 || t->k_stride_tok % 8)
    return fail(BSK_ERR_INVALID_ARG, "strides must be multiples of 16 bytes");
  const int64_t max_visible = problem->window > 0 ? std::min<int64_t>(max_kv_len, int64_t(problem->window) + problem->sink)
                                                  : max_kv_len;
  const int64_t need = problem->rope_mode == BSK_ROPE_STREAMING ? max_visible : max_kv_len;
  if (t->rope_n_pos < need) return fail(BSK_ERR_INVALID_ARG, "rope table has too few positions");
  bsk::RopeApplyArgs a;
  a.q = t->q;
  a.q_st = t->q_stride_tok;
  a.q_sh = t->q_stride_head;
  a.q_out = q_out;
  a.qo_st = qo_stride_tok;
  a.qo_sh = qo_stride_head;
  a.k = t->k;
  a.k_out = k_out;
  a.k_sp = t->k_stride_page;
  a.k_sh = t->k_stride_head;
  a.k_st = t->k_stride_tok;
  a.qo_indptr = qo_indptr;
  a.kv_len = kv_len;
  a.page_indptr = kv_page_indptr;
  a.page_indices = t->kv_page_indices;
  a.rope = t->rope_cos_sin;
  a.rope_n_pos = t->rope_n_pos;
  a.batch = batch;
  a.num_qo_heads = problem->num_qo_heads;
  a.num_kv_heads = problem->num_kv_heads;
  a.page_shift = ilog2(problem->page_size);
  a.window = problem->window > 0 ? problem->window : 0;
  a.sink = problem->window > 0 ? problem->sink : 0;
  a.streaming = problem->rope_mode == BSK_ROPE_STREAMING;
  hipError_t e = bsk::launch_rope_apply(problem->head_dim, a, int(max_visible), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope apply launch");
  return BSK_OK;
}

bsk_status bsk_debug_gather(const bsk_problem* problem, const bsk_plan_info* info, const bsk_tensors* t,
                            const void* int_ws_dev, const int64_t* row_offsets, void* k_out, void* v_out,
                            void* stream) {
  bsk_status s = check_problem(problem);
  if (s != BSK_OK) return s;
  if (!info || !t || !int_ws_dev || !row_offsets || !k_out || !v_out || !t->k || !t->v)
    return fail(BSK_ERR_INVALID_ARG, "null argument");
  if (problem->kv_mode == BSK_KV_PAGED && !t->kv_page_indices) return fail(BSK_ERR_INVALID_ARG, "kv_page_indices");
  const bsk::AttnArgs a = attn_args(*problem, *t, int_ws_dev, nullptr);
  hipError_t e = bsk::launch_gather(problem->dtype, problem->head_dim, problem->kv_mode == BSK_KV_DENSE, a,
                                    row_offsets, k_out, v_out, info->num_workers, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return BSK_OK;
}

bsk_status bsk_debug_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, int32_t grid,
                                 void* stream) {
  if (!src || !sink) return fail(BSK_ERR_INVALID_ARG, "null argument");
  if (!aligned(src, 16) || bytes % 16 != 0) return fail(BSK_ERR_INVALID_ARG, "src must be 16-byte aligned, bytes a multiple of 16");
  if (grid <= 0 || grid > (1 << 20)) return fail(BSK_ERR_INVALID_ARG, "grid must be in [1, 2^20]");
  if (!aligned(sink, 4) || sink_bytes < size_t(grid) * size_t(bsk::stream_read_threads()) * sizeof(uint32_t))
    return fail(BSK_ERR_INVALID_ARG, "sink must hold one 32-bit word per thread (grid * 256)");
  hipError_t e = bsk::launch_stream_read(src, int64_t(bytes / 16), static_cast<uint32_t*>(sink), grid,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream read launch");
  return BSK_OK;
}

bsk_status bsk_debug_block_read(const void* src, size_t bytes, const int32_t* order, int32_t n_blocks, void* sink,
                                size_t sink_bytes, int32_t grid, void* stream) {
  if (!src || !order || !sink) return fail(BSK_ERR_INVALID_ARG, "null argument");
  if (!aligned(src, 16) || bytes < 4096 || bytes % 4096 != 0)
    return fail(BSK_ERR_INVALID_ARG, "src must be 16-byte aligned, bytes a positive multiple of 4096");
  if (!aligned(order, 4) || n_blocks <= 0) return fail(BSK_ERR_INVALID_ARG, "order must be int32-aligned, n_blocks > 0");
  if (grid <= 0 || grid > (1 << 20)) return fail(BSK_ERR_INVALID_ARG, "grid must be in [1, 2^20]");
  if (!aligned(sink, 4) || sink_bytes < size_t(grid) * size_t(bsk::stream_read_threads()) * sizeof(uint32_t))
    return fail(BSK_ERR_INVALID_ARG, "sink must hold one 32-bit word per thread (grid * 256)");
  hipError_t e = bsk::launch_block_read(src, int64_t(bytes / 4096), order, n_blocks, static_cast<uint32_t*>(sink),
                                        grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "block read launch");
  return BSK_OK;
}

}  // extern "C"
#pragma GCC visibility pop
