// Large-tile persistent attention kernel (128 query rows per work item).
//
// Serves ragged causal prefill, including prefill appended after cached KV
// (FlashInfer 0.6 wiki, "Kernel types": Prefill, compute-bound, chunked
// prefill) and the dense shared prefix of the composable format (FlashInfer
// paper summary, "Research methodology" 1), where all branch queries of a
// kv head form one tile and read the prefix once.  Same persistent
// plan-driven structure as the small-tile kernel; bf16 only.
//
// Per item (request r, kv head h, rows [row_lo, row_lo + 128), keys
// [kv_lo, kv_hi)): each of the four waves owns 32 rows (two 16-row MFMA
// column blocks) and the whole key range.  Keys go through LDS in 64-key
// tiles -- K and V rows are copied with coalesced 16-byte loads, the next
// tile's loads are issued before the current tile is consumed --
//   S^T (64 x 32) = K Q^T    16x16x32 bf16 MFMA, K from LDS, q in registers
//   online softmax in base 2, fp32
//   O^T (D x 32) += V^T P^T  16x16x32 bf16 MFMA, V read key-major from LDS
// and every wave writes its own rows (output or partial state).

#include "device.h"
#include "launch.h"

namespace bsk {

constexpr int kPreRows = 128;
constexpr int kPreWaves = 4;
constexpr int kPreThreads = kPreWaves * kWave;
constexpr int kPreKeys = 64;  // keys per LDS tile

template <int D, bool DENSE>
__global__ __launch_bounds__(kPreThreads, 2) void prefill_kernel(AttnArgs a) {
  constexpr int ROW = D + 8;            // bf16 per LDS row (padding spreads banks)
  constexpr int NKS = D / 32;           // k-steps over d for the logits
  constexpr int NDB = D / 16;           // 16-wide output column blocks
  constexpr int CPR = D / 8;            // 16-byte chunks per key row
  constexpr int KPP = kPreThreads / CPR;  // key rows per load pass
  constexpr int NPASS = kPreKeys / KPP;   // load passes per tile
  static_assert(D == 64 || D == 128, "head_dim");

  __shared__ __align__(16) unsigned short s_k[kPreKeys * ROW];
  __shared__ __align__(16) unsigned short s_v[kPreKeys * ROW];
  __shared__ int32_t s_pages[DENSE ? 1 : kMaxPages];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int j = lane >> 4;
  const int lc = tid % CPR;  // load assignment: chunk of a key row
  const int lk = tid / CPR;  // and the key row (plus multiples of KPP)

  const int32_t* __restrict__ ws = a.ws;
  const int it_begin = ws[HDR_WORDS + blockIdx.x];
  const int it_end = ws[HDR_WORDS + blockIdx.x + 1];
  const int32_t* __restrict__ items = ws + ws[HDR_OFF_ITEMS];
  const int32_t* __restrict__ qo_indptr = ws + ws[HDR_OFF_QO];
  const int32_t* __restrict__ kv_lens = ws + ws[HDR_OFF_KVLEN];
  const int32_t* __restrict__ kv_ind = ws + ws[HDR_OFF_KVIND];
  const __bf16* __restrict__ Qp = static_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ Kp = static_cast<const __bf16*>(a.k);
  const __bf16* __restrict__ Vp = static_cast<const __bf16*>(a.v);
  const int g = a.group;

  for (int it = it_begin; it < it_end; ++it) {
    const int32_t* rec = items + int64_t(it) * ITEM_WORDS;
    const int r = rec[IT_R], h = rec[IT_H];
    const int row_lo = rec[IT_ROW_LO], row_hi = rec[IT_ROW_HI];
    const int kv_lo = rec[IT_KV_LO], kv_hi = rec[IT_KV_HI];
    const int slot = rec[IT_SLOT];
    const int q0 = qo_indptr[r];
    const int qlen = qo_indptr[r + 1] - q0;
    const int L = kv_lens[r];
    const int kbase = kv_ind[r];

    if constexpr (!DENSE) stage_pages(s_pages, a.page_indices, kbase, kv_lo, kv_hi, a.page_shift, tid, kPreThreads);
    __syncthreads();

    // this lane's two query rows (one per 16-row column block) and q fragments
    int qpos[2];
    bool row_ok[2];
    bf16x8 qf[2][NKS];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int row = row_lo + 32 * wave + 16 * nb + n;
      row_ok[nb] = row < row_hi;
      const int qi = row_ok[nb] ? row / g : 0;
      const int qu = row_ok[nb] ? row % g : 0;
      qpos[nb] = L - qlen + qi;
      const __bf16* qrow = Qp + int64_t(q0 + qi) * a.q_st + int64_t(h * g + qu) * a.q_sh;
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        qf[nb][s] = row_ok[nb] ? *reinterpret_cast<const bf16x8*>(qrow + 8 * (4 * s + j)) : bf16x8{};
    }

    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    f32x4 acc[2][NDB];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[nb][db] = f32x4{0, 0, 0, 0};

    bf16x8 kreg[NPASS], vreg[NPASS];
    auto load_tile = [&](int kt) {
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        const int t = min(kt + lk + p * KPP, kv_hi - 1);
        const int64_t ko = kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.k_sp, a.k_sh, a.k_st);
        const int64_t vo = kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.v_sp, a.v_sh, a.v_st);
        kreg[p] = *reinterpret_cast<const bf16x8*>(Kp + ko + 8 * lc);
        vreg[p] = *reinterpret_cast<const bf16x8*>(Vp + vo + 8 * lc);
      }
    };

    const int ntiles = (kv_hi - kv_lo + kPreKeys - 1) / kPreKeys;
    load_tile(kv_lo);
    for (int tile = 0; tile < ntiles; ++tile) {
      const int kt = kv_lo + tile * kPreKeys;
      __syncthreads();
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        *reinterpret_cast<bf16x8*>(s_k + (lk + p * KPP) * ROW + 8 * lc) = kreg[p];
        *reinterpret_cast<bf16x8*>(s_v + (lk + p * KPP) * ROW + 8 * lc) = vreg[p];
      }
      __syncthreads();
      if (tile + 1 < ntiles) load_tile(kt + kPreKeys);

      // S^T[key][row] for 4 key blocks x 2 row blocks
      f32x4 st[4][2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) st[mb][0] = st[mb][1] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(s_k + (16 * mb + n) * ROW + 8 * (4 * s + j));
          st[mb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][s], st[mb][0], 0, 0, 0);
          st[mb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][s], st[mb][1], 0, 0, 0);
        }
      }

      // mask, online softmax, P^T operands
      bf16x8 pb[2][2];  // [row block][32-key step]
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float sv[4][4];
        float bm = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = kt + 16 * mb + 4 * j + i;
            const bool ok = row_ok[nb] && t < kv_hi && key_visible(t, qpos[nb], a.causal, a.window, a.sink);
            sv[mb][i] = ok ? st[mb][nb][i] * a.scale_log2 : -INFINITY;
            bm = fmaxf(bm, sv[mb][i]);
          }
        bm = wave_max_xor16_32(bm);
        const float m_new = fmaxf(m_run[nb], bm);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[nb] - m_use);
        float psum = 0.f;
        u32x4 pw[2];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = __builtin_amdgcn_exp2f(sv[mb][i] - m_use);
            psum += p[i];
          }
          // key step ks = mb / 2 holds blocks 2ks (elements 0..3) and 2ks+1 (elements 4..7)
          pw[mb >> 1][(mb & 1) * 2] = pack_bf16x2(p[0], p[1]);
          pw[mb >> 1][(mb & 1) * 2 + 1] = pack_bf16x2(p[2], p[3]);
        }
        pb[nb][0] = __builtin_bit_cast(bf16x8, pw[0]);
        pb[nb][1] = __builtin_bit_cast(bf16x8, pw[1]);
        l_run[nb] = l_run[nb] * alpha + psum;
        m_run[nb] = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[nb][db] *= alpha;
      }

      // O^T[d][row] += V^T P^T; MFMA k index 8j+e maps to key 32ks + 4j + (e&3) + 16(e>>2)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          u32x4 vw;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int e0 = 2 * e2, e1 = 2 * e2 + 1;
            const int k0 = 32 * ks + 4 * j + (e0 & 3) + 16 * (e0 >> 2);
            const int k1 = 32 * ks + 4 * j + (e1 & 3) + 16 * (e1 >> 2);
            vw[e2] = uint32_t(s_v[k0 * ROW + 16 * db + n]) | (uint32_t(s_v[k1 * ROW + 16 * db + n]) << 16);
          }
          const bf16x8 va = __builtin_bit_cast(bf16x8, vw);
          acc[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[0][ks], acc[0][db], 0, 0, 0);
          acc[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[1][ks], acc[1][db], 0, 0, 0);
        }
      }
    }

    // epilogue: each lane owns row n of each row block, columns 16db + 4j + i
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float lsum = wave_sum_xor16_32(l_run[nb]);
      if (!row_ok[nb]) continue;
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      const float lse = lsum > 0.f ? (m_run[nb] + __log2f(lsum)) * 0.69314718055994531f : -INFINITY;
      const int rr = 32 * wave + 16 * nb + n;  // row within the tile
      const int row = row_lo + rr;
      if (slot < 0) {
        const int tok = q0 + row / g;
        const int qhd = h * g + row % g;
        const int64_t ob = int64_t(tok) * a.o_st + int64_t(qhd) * a.o_sh;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const f32x4 o = acc[nb][db] * inv;
          const int64_t oo = ob + 16 * db + 4 * j;
          if (a.out_bf16) {
            uint2 pk2 = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            *reinterpret_cast<uint2*>(static_cast<__bf16*>(a.out) + oo) = pk2;
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + oo) = float4{o[0], o[1], o[2], o[3]};
          }
        }
        if (j == 0) a.lse[int64_t(tok) * a.lse_st + qhd] = lse;
      } else {
        float* po = a.part_o + (int64_t(slot) * kPreRows + rr) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const f32x4 o = acc[nb][db] * inv;
          *reinterpret_cast<float4*>(po + 16 * db + 4 * j) = float4{o[0], o[1], o[2], o[3]};
        }
        if (j == 0) a.part_lse[int64_t(slot) * kPreRows + rr] = lse;
      }
    }
    if (slot >= 0 && a.fused_merge) finish_split_chunk<D>(a, slot, tid, kPreThreads, &s_last);
  }
}

hipError_t launch_prefill(int head_dim, bool dense, const AttnArgs& a, int grid, hipStream_t stream) {
#define BSK_PRE(D, DN)                                                                                      \
  if (head_dim == D && dense == DN) {                                                                       \
    hipLaunchKernelGGL((prefill_kernel<D, DN>), dim3(grid), dim3(kPreThreads), 0, stream, a);              \
    return hipGetLastError();                                                                               \
  }
  BSK_PRE(128, false)
  BSK_PRE(128, true)
  BSK_PRE(64, false)
  BSK_PRE(64, true)
#undef BSK_PRE
  return hipErrorInvalidValue;
}

const void* prefill_kernel_ptr(int head_dim, bool dense) {
  if (head_dim == 128) return dense ? reinterpret_cast<const void*>(&prefill_kernel<128, true>)
                                    : reinterpret_cast<const void*>(&prefill_kernel<128, false>);
  if (head_dim == 64) return dense ? reinterpret_cast<const void*>(&prefill_kernel<64, true>)
                                   : reinterpret_cast<const void*>(&prefill_kernel<64, false>);
  return nullptr;
}

int prefill_threads() { return kPreThreads; }

}  // namespace bsk
