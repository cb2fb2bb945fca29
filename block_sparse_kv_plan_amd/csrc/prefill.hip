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
// tiles, double-buffered: the next tile's rows are fetched into registers
// with coalesced 16-byte loads while the current tile is consumed, then
// stored to the other buffer, so one barrier per tile suffices.
//   S^T (64 x 32) = K Q^T    16x16x32 bf16 MFMA, K from LDS, q in registers
//   online softmax in base 2, fp32; masks are evaluated only on tiles that
//   cross a boundary (range end, causal diagonal, window); the accumulator
//   is rescaled only when a row's max grows by more than 2^8
//   O^T (D x 32) += V^T P^T  16x16x32 bf16 MFMA; each lane reads whole
//   16-byte pieces of eight V rows and repacks them, the MFMA key index
//   being mapped to the keys whose probabilities the lane already holds
// and every wave writes its own rows (output or partial state).

#include "device.h"
#include "launch.h"

namespace bsk {

constexpr int kPreRows = 128;
constexpr int kPreWaves = 4;
constexpr int kPreThreads = kPreWaves * kWave;
constexpr int kPreKeys = 64;                  // keys per LDS tile
constexpr float kPreRescaleSlack = 8.f;       // log2 units

// Element e of eight 8-element pieces, as an MFMA k-octet (pieces 0..7 -> k 0..7).
__device__ __forceinline__ bf16x8 gather8(const u32x4* v, int e) {
  const int w = e >> 1;
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = __builtin_amdgcn_perm(v[2 * q + 1][w], v[2 * q][w], sel);
  return __builtin_bit_cast(bf16x8, r);
}

template <int D, bool DENSE>
__global__ __launch_bounds__(kPreThreads, 2) void prefill_kernel(AttnArgs a) {
  constexpr int ROW = D + 8;              // bf16 per LDS row (padding spreads banks)
  constexpr int NKS = D / 32;             // k-steps over d for the logits
  constexpr int CHUNKS = D / 8;           // 16-byte pieces per row
  constexpr int CPR = D / 8;              // load assignment: pieces per key row
  constexpr int KPP = kPreThreads / CPR;  // key rows per load pass
  constexpr int NPASS = kPreKeys / KPP;   // load passes per tile
  constexpr int TILE_ELEMS = kPreKeys * ROW;
  static_assert(D == 64 || D == 128, "head_dim");

  __shared__ __align__(16) unsigned short s_k[2 * TILE_ELEMS];
  __shared__ __align__(16) unsigned short s_v[2 * TILE_ELEMS];
  __shared__ int32_t s_pages[DENSE ? 1 : kMaxPages];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int j = lane >> 4;
  const int lc = tid % CPR;  // load assignment: piece of a key row
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
    // the wave's query-position range (rows past row_hi excluded), for the mask-free test
    const int wrow0 = row_lo + 32 * wave;
    const int wrow1 = min(row_hi, wrow0 + 32) - 1;  // may be < wrow0 for an empty wave
    const int wq_lo = L - qlen + (wrow0 < row_hi ? wrow0 / g : 0);
    const int wq_hi = L - qlen + (wrow1 >= wrow0 ? wrow1 / g : 0);
    const bool wave_has_rows = wrow0 < row_hi;
    const bool all_rows = wrow0 + 32 <= row_hi;

    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    f32x4 acc[2][8];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[nb][e] = f32x4{0, 0, 0, 0};

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
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        *reinterpret_cast<bf16x8*>(s_k + buf * TILE_ELEMS + (lk + p * KPP) * ROW + 8 * lc) = kreg[p];
        *reinterpret_cast<bf16x8*>(s_v + buf * TILE_ELEMS + (lk + p * KPP) * ROW + 8 * lc) = vreg[p];
      }
    };

    const int ntiles = (kv_hi - kv_lo + kPreKeys - 1) / kPreKeys;
    load_tile(kv_lo);
    store_tile(0);
    __syncthreads();
    for (int tile = 0; tile < ntiles; ++tile) {
      const int kt = kv_lo + tile * kPreKeys;
      const int buf = tile & 1;
      const bool more = tile + 1 < ntiles;
      if (more) load_tile(kt + kPreKeys);  // in flight during this tile's math
      const unsigned short* sk = s_k + buf * TILE_ELEMS;
      const unsigned short* sv = s_v + buf * TILE_ELEMS;

      if (wave_has_rows) {
        // S^T[key][row] for 4 key blocks x 2 row blocks
        f32x4 st[4][2];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) st[mb][0] = st[mb][1] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sk + (16 * mb + n) * ROW + 8 * (4 * s + j));
            st[mb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][s], st[mb][0], 0, 0, 0);
            st[mb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][s], st[mb][1], 0, 0, 0);
          }
        }

        // masks only where the tile crosses a boundary for some row of this wave
        const int kend = kt + kPreKeys - 1;
        bool clean = all_rows && kend < kv_hi;
        if (a.causal) clean = clean && kend <= wq_lo;
        if (a.window > 0) clean = clean && (wq_hi - kt) < a.window;
        bf16x8 pb[2][2];  // [row block][32-key step]
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if (!clean) {
            const RowMask rm = row_mask(row_ok[nb], qpos[nb], kv_hi, a.causal, a.window, a.sink);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                st[mb][nb][i] = row_sees(rm, kt + 16 * mb + 4 * j + i) ? st[mb][nb][i] : -INFINITY;
          }
          float bm = -INFINITY;
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            bm = fmaxf(bm, fmaxf(fmaxf(st[mb][nb][0], st[mb][nb][1]), fmaxf(st[mb][nb][2], st[mb][nb][3])));
          bm = wave_max_xor16_32(bm) * a.scale_log2;  // scale > 0 keeps the max
          const bool grow = bm > m_run[nb] + kPreRescaleSlack || (m_run[nb] == -INFINITY && bm > -INFINITY);
          if (__any(grow)) {
            const float m_new = grow ? bm : m_run[nb];
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[nb] - m_new);
            l_run[nb] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[nb][e] *= alpha;
            m_run[nb] = m_new;
          }
          const float neg_m = m_run[nb] == -INFINITY ? 0.f : -m_run[nb];
          float psum = 0.f;
          u32x4 pw[2];
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[mb][nb][i], a.scale_log2, neg_m));
              psum += p[i];
            }
            // key step ks = mb / 2 holds blocks 2ks (elements 0..3) and 2ks+1 (elements 4..7)
            pw[mb >> 1][(mb & 1) * 2] = pack_bf16x2(p[0], p[1]);
            pw[mb >> 1][(mb & 1) * 2 + 1] = pack_bf16x2(p[2], p[3]);
          }
          pb[nb][0] = __builtin_bit_cast(bf16x8, pw[0]);
          pb[nb][1] = __builtin_bit_cast(bf16x8, pw[1]);
          l_run[nb] += psum;
        }

        // O^T[d][row] += V^T P^T.  MFMA k index 8j+e <-> key 32ks + 4j + (e&3) + 16(e>>2): the keys
        // whose probabilities this lane holds.  The lane reads piece n % CHUNKS of those eight V
        // rows; MFMA number e then covers columns d = 8 (n % CHUNKS) + e.
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4 vrow[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = 32 * ks + 4 * j + (e & 3) + 16 * (e >> 2);
            vrow[e] = *reinterpret_cast<const u32x4*>(sv + key * ROW + 8 * (n % CHUNKS));
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bf16x8 va = gather8(vrow, e);
            acc[0][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[0][ks], acc[0][e], 0, 0, 0);
            acc[1][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[1][ks], acc[1][e], 0, 0, 0);
          }
        }
      }
      if (more) store_tile(buf ^ 1);  // the other buffer was last read before the previous barrier
      __syncthreads();
    }

    // epilogue: each lane owns row n of each row block; acc[nb][e][i] is column 8 (4j+i) + e
    // (with D = 64, lane groups j >= 2 repeat j - 2 and do not write)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float lsum = wave_sum_xor16_32(l_run[nb]);
      if (!row_ok[nb]) continue;
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      const float lse = lsum > 0.f ? (m_run[nb] + __log2f(lsum)) * 0.69314718055994531f : -INFINITY;
      const int rr = 32 * wave + 16 * nb + n;  // row within the tile
      const int row = row_lo + rr;
      float* po = nullptr;
      int64_t ob = 0;
      if (slot < 0) {
        const int tok = q0 + row / g;
        const int qhd = h * g + row % g;
        ob = int64_t(tok) * a.o_st + int64_t(qhd) * a.o_sh;
        if (j == 0) a.lse[int64_t(tok) * a.lse_st + qhd] = lse;
      } else {
        po = a.part_o + (int64_t(slot) * kPreRows + rr) * D;
        if (j == 0) a.part_lse[int64_t(slot) * kPreRows + rr] = lse;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 4 * j + i;
        if (c >= CHUNKS) continue;
        const float4 o0 = {acc[nb][0][i] * inv, acc[nb][1][i] * inv, acc[nb][2][i] * inv, acc[nb][3][i] * inv};
        const float4 o1 = {acc[nb][4][i] * inv, acc[nb][5][i] * inv, acc[nb][6][i] * inv, acc[nb][7][i] * inv};
        if (slot < 0) {
          const int64_t oo = ob + 8 * c;
          if (a.out_bf16) {
            uint4 pk = {pack_bf16x2(o0.x, o0.y), pack_bf16x2(o0.z, o0.w), pack_bf16x2(o1.x, o1.y),
                        pack_bf16x2(o1.z, o1.w)};
            *reinterpret_cast<uint4*>(static_cast<__bf16*>(a.out) + oo) = pk;
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + oo) = o0;
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + oo + 4) = o1;
          }
        } else {
          *reinterpret_cast<float4*>(po + 8 * c) = o0;
          *reinterpret_cast<float4*>(po + 8 * c + 4) = o1;
        }
      }
    }
    if (slot >= 0 && a.fused_merge) finish_split_chunk<D>(a, slot, tid, kPreThreads, &s_last);
  }
}

hipError_t launch_prefill(int head_dim, bool dense, const AttnArgs& a, int grid, hipStream_t stream) {
#define BSK_PRE(D, DN)                                                                         \
  if (head_dim == D && dense == DN) {                                                          \
    hipLaunchKernelGGL((prefill_kernel<D, DN>), dim3(grid), dim3(kPreThreads), 0, stream, a); \
    return hipGetLastError();                                                                  \
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
