// Large-tile persistent attention kernel (128 or 256 query rows per work item).
//
// Serves ragged causal prefill, including prefill appended after cached KV
// (FlashInfer 0.6 wiki, "Kernel types": Prefill, compute-bound, chunked
// prefill) and the dense shared prefix of the composable format (FlashInfer
// paper summary, "Research methodology" 1), where all branch queries of a
// kv head form one tile and read the prefix once.  Same persistent
// plan-driven structure as the small-tile kernel; bf16 only.
//
// Per item (request r, kv head h, rows [row_lo, row_lo + 64 NB), keys
// [kv_lo, kv_hi)): each of the four waves owns 16 NB rows (NB 16-row MFMA
// column blocks) and the whole key range.  Keys go through LDS in 64-key
// tiles, double-buffered: the next tile's rows are fetched into registers
// with coalesced 16-byte loads while the current tile is consumed, then
// stored to the other buffer, so one barrier per tile suffices.
//   S^T (64 x 16 NB) = K Q^T    16x16x32 bf16 MFMA, K from LDS, q in registers
//   online softmax in base 2, fp32; masks are evaluated only on tiles that
//   cross a boundary (range end, causal diagonal, window); the accumulator
//   is rescaled only when a row's max grows by more than 2^8
//   O^T (D x 16 NB) += V^T P^T  16x16x32 bf16 MFMA; each lane reads whole
//   16-byte pieces of eight V rows and repacks them, the MFMA key index
//   being mapped to the keys whose probabilities the lane already holds
// and every wave writes its own rows (output or partial state).
//
// Every K/V tile read from LDS is shared by all NB row blocks of a wave, so
// NB = 4 (64 rows per wave, one workgroup per CU with up to 512 registers
// per lane) halves the LDS reads, V repacks and address work per MFMA
// relative to NB = 2 (32 rows per wave, two workgroups per CU).
//
// The logit max uses fmaxf on values that are never NaN (masked logits are
// replaced by -inf before it), so this file is built without NaN semantics
// and the max needs no operand canonicalisation.

#include "device.h"
#include "launch.h"

namespace bsk {

constexpr int kPreWaves = 4;
constexpr int kPreThreads = kPreWaves * kWave;
constexpr int kPreKeys = 64;                  // keys per LDS tile
constexpr float kPreRescaleSlack = 8.f;       // log2 units

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

// Two transposing 8-byte LDS reads (ds_read_b64_tr_b16) joined into one MFMA k-octet.  Within
// each 16-lane group the instruction gathers the 4 x 16-bit values each lane points at and hands
// lane i element i % 4 of the values addressed by lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4.
__device__ __forceinline__ bf16x8 ds_read_tr_pair(const unsigned short* p0, const unsigned short* p1) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D, bool DENSE, int NB>
__global__ __launch_bounds__(kPreThreads, NB <= 2 ? 2 : 1) void prefill_kernel(AttnArgs a) {
  constexpr int ROWS = kPreWaves * 16 * NB;  // query rows per item (the plan's tile_q)
  constexpr int WROWS = 16 * NB;             // rows per wave
  constexpr int ROW = D + 8;                 // bf16 per K row in LDS (padding spreads banks for
                                             // the 16-byte row reads)
  constexpr int ROWV = D + 16;               // bf16 per V row (spreads banks for the transposing reads)
  constexpr int NDB = D / 16;                // 16-column blocks of the output
  constexpr int NKS = D / 32;                // k-steps over d for the logits
  constexpr int CHUNKS = D / 8;              // 16-byte pieces per row
  constexpr int KPP = kPreThreads / CHUNKS;  // key rows per load pass
  constexpr int NPASS = kPreKeys / KPP;      // load passes per tile
  constexpr int TILE_ELEMS = kPreKeys * ROW;
  constexpr int TILE_ELEMS_V = kPreKeys * ROWV;
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(NB == 2 || NB == 4, "row blocks per wave");

  __shared__ __align__(16) unsigned short s_k[2 * TILE_ELEMS];
  __shared__ __align__(16) unsigned short s_v[2 * TILE_ELEMS_V];
  __shared__ int32_t s_pages[DENSE ? 1 : kMaxPages];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int j = lane >> 4;
  const int lc = tid % CHUNKS;  // load assignment: piece of a key row
  const int lk = tid / CHUNKS;  // and the key row (plus multiples of KPP)

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
  const int pmask = (1 << a.page_shift) - 1;
  // page strides in bytes; the host checks that they fit 32 bits
  const uint32_t k_page_bytes = uint32_t(a.k_sp) * 2u;
  const uint32_t v_page_bytes = uint32_t(a.v_sp) * 2u;

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

    // this lane's query rows (one per 16-row column block) and q fragments
    int qpos[NB];
    bool row_ok[NB];
    bf16x8 qf[NB][NKS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int row = row_lo + WROWS * wave + 16 * nb + n;
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
    const int wrow0 = row_lo + WROWS * wave;
    const int wrow1 = min(row_hi, wrow0 + WROWS) - 1;  // may be < wrow0 for an empty wave
    const int wq_lo = L - qlen + (wrow0 < row_hi ? wrow0 / g : 0);
    const int wq_hi = L - qlen + (wrow1 >= wrow0 ? wrow1 / g : 0);
    const bool wave_has_rows = wrow0 < row_hi;
    const bool all_rows = wrow0 + WROWS <= row_hi;

    float m_run[NB], l_run[NB];
    f32x4 acc[NB][NDB];  // acc[nb][db][i] = O^T[16 db + 4 j + i][row n of block nb]
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = -INFINITY;
      l_run[nb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[nb][db] = f32x4{0, 0, 0, 0};
    }

    // Load addressing.  Thread (lk, lc) fetches piece lc of key rows lk + p KPP of each tile.
    // When tiles start at multiples of 64 keys (always for dense KV; for paged KV when the item
    // does), a full tile's row p sits in page slot (kt >> shift) - p0 + slot_p at in-page token
    // (kt & pmask) + (r_p & pmask): a page of <= 64 keys divides the tile, a larger page holds all
    // of it.  Then the address is one 32 x 32 -> 64-bit multiply-add of the page id.
    const bool fast_item = DENSE || (kv_lo & (kPreKeys - 1)) == 0;
    // 32-bit part of each row's address that does not change from tile to tile: head, in-page
    // token (paged) or tile-relative token (dense), and the 16-byte piece.  It is below the page
    // stride (paged) or below 2^32 for dense blocks the host accepts.
    uint32_t koff[NPASS], voff[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int rr = lk + p * KPP;
      const int tok = DENSE ? rr : (rr & pmask);
      koff[p] = uint32_t(2 * (int64_t(h) * a.k_sh + int64_t(tok) * a.k_st + 8 * lc));
      voff[p] = uint32_t(2 * (int64_t(h) * a.v_sh + int64_t(tok) * a.v_st + 8 * lc));
    }
    const int p0 = kv_lo >> a.page_shift;

    bf16x8 kreg[NPASS], vreg[NPASS];
    auto load_tile = [&](int kt) {
      if (fast_item && kt + kPreKeys <= kv_hi) {
        if constexpr (DENSE) {
          const char* kb = reinterpret_cast<const char*>(Kp) + 2 * (int64_t(kbase + kt) * a.k_st);
          const char* vb = reinterpret_cast<const char*>(Vp) + 2 * (int64_t(kbase + kt) * a.v_st);
#pragma unroll
          for (int p = 0; p < NPASS; ++p) {
            kreg[p] = *reinterpret_cast<const bf16x8*>(kb + koff[p]);
            vreg[p] = *reinterpret_cast<const bf16x8*>(vb + voff[p]);
          }
        } else {
          const int sb = (kt >> a.page_shift) - p0;
          const char* kb = reinterpret_cast<const char*>(Kp) + 2 * (int64_t(kt & pmask) * a.k_st);
          const char* vb = reinterpret_cast<const char*>(Vp) + 2 * (int64_t(kt & pmask) * a.v_st);
#pragma unroll
          for (int p = 0; p < NPASS; ++p) {
            const uint32_t page = uint32_t(s_pages[sb + ((lk + p * KPP) >> a.page_shift)]);
            kreg[p] = *reinterpret_cast<const bf16x8*>(kb + (uint64_t(page) * k_page_bytes + koff[p]));
            vreg[p] = *reinterpret_cast<const bf16x8*>(vb + (uint64_t(page) * v_page_bytes + voff[p]));
          }
        }
      } else {
        // ragged tail or unaligned start: clamp rows past the range to the last key
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
          const int t = min(kt + lk + p * KPP, kv_hi - 1);
          const int64_t ko = kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.k_sp, a.k_sh, a.k_st);
          const int64_t vo = kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.v_sp, a.v_sh, a.v_st);
          kreg[p] = *reinterpret_cast<const bf16x8*>(Kp + ko + 8 * lc);
          vreg[p] = *reinterpret_cast<const bf16x8*>(Vp + vo + 8 * lc);
        }
      }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        *reinterpret_cast<bf16x8*>(s_k + buf * TILE_ELEMS + (lk + p * KPP) * ROW + 8 * lc) = kreg[p];
        *reinterpret_cast<bf16x8*>(s_v + buf * TILE_ELEMS_V + (lk + p * KPP) * ROWV + 8 * lc) = vreg[p];
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
      const unsigned short* sv = s_v + buf * TILE_ELEMS_V;

      if (wave_has_rows) {
        // masks only where the tile crosses a boundary for some row of this wave
        const int kend = kt + kPreKeys - 1;
        bool clean = all_rows && kend < kv_hi;
        if (a.causal) clean = clean && kend <= wq_lo;
        if (a.window > 0) clean = clean && (wq_hi - kt) < a.window;
        // two 32-key halves, each: logits, softmax, PV (halves the live logit registers)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          // S^T[key][row] for key blocks 2ks, 2ks+1 x NB row blocks
          f32x4 st[2][NB];
#pragma unroll
          for (int mh = 0; mh < 2; ++mh)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) st[mh][nb] = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int s = 0; s < NKS; ++s) {
#pragma unroll
            for (int mh = 0; mh < 2; ++mh) {
              const int mb = 2 * ks + mh;
              const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sk + (16 * mb + n) * ROW + 8 * (4 * s + j));
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)
                st[mh][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[nb][s], st[mh][nb], 0, 0, 0);
            }
          }
          if (!clean) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              const RowMask rm = row_mask(row_ok[nb], qpos[nb], kv_hi, a.causal, a.window, a.sink);
#pragma unroll
              for (int mh = 0; mh < 2; ++mh)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  st[mh][nb][i] = row_sees(rm, kt + 16 * (2 * ks + mh) + 4 * j + i) ? st[mh][nb][i] : -INFINITY;
            }
          }
          // Online softmax with a lazily moved reference: each lane checks its own logits against
          // the row's reference plus the slack; only if some lane exceeds it is the row max
          // reduced across the row's four lanes and the state rescaled.
          float lmax[NB];
          bool grow = false;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            lmax[nb] = fmaxf(fmaxf(fmaxf(st[0][nb][0], st[0][nb][1]), fmaxf(st[0][nb][2], st[0][nb][3])),
                             fmaxf(fmaxf(st[1][nb][0], st[1][nb][1]), fmaxf(st[1][nb][2], st[1][nb][3])));
            grow = grow || lmax[nb] * a.scale_log2 > m_run[nb] + kPreRescaleSlack;
          }
          if (__any(grow)) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              const float bm = wave_max_xor16_32(lmax[nb]) * a.scale_log2;  // scale > 0 keeps the max
              if (bm > m_run[nb] + kPreRescaleSlack) {
                const float alpha = m_run[nb] == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[nb] - bm);
                l_run[nb] *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) acc[nb][db] *= alpha;
                m_run[nb] = bm;
              }
            }
          }
          bf16x8 pb[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const float neg_m = m_run[nb] == -INFINITY ? 0.f : -m_run[nb];
            float psum = 0.f;
            u32x4 pw;
#pragma unroll
            for (int mh = 0; mh < 2; ++mh) {
              float pr[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[mh][nb][i], a.scale_log2, neg_m));
                psum += pr[i];
              }
              // MFMA k elements 0..3 hold key block 2ks, elements 4..7 block 2ks+1
              pw[2 * mh] = pack_bf16x2(pr[0], pr[1]);
              pw[2 * mh + 1] = pack_bf16x2(pr[2], pr[3]);
            }
            pb[nb] = __builtin_bit_cast(bf16x8, pw);
            l_run[nb] += psum;
          }

          // O^T[d][row] += V^T P^T.  MFMA k index 8j+e <-> key 32ks + 4j + (e&3) + 16(e>>2): the
          // keys whose probabilities this lane holds.  The V^T operand comes from two transposing
          // LDS reads: in each 16-lane group, lane k points at 4 columns of key row k/4 and gets
          // back one column of 4 keys, so lane (n, j) receives V[key(8j+e)][16 db + n].
          {
            const unsigned short* vb = sv + (32 * ks + 4 * j + (n >> 2)) * ROWV + 4 * (n & 3);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const bf16x8 va = ds_read_tr_pair(vb + 16 * db, vb + 16 * db + 16 * ROWV);
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)
                acc[nb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[nb], acc[nb][db], 0, 0, 0);
            }
          }
        }
      }
      if (more) store_tile(buf ^ 1);  // the other buffer was last read before the previous barrier
      __syncthreads();
    }

    // epilogue: each lane owns row n of each row block and columns 16 db + 4 j .. + 3
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float lsum = wave_sum_xor16_32(l_run[nb]);
      if (!row_ok[nb]) continue;
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      const float lse = lsum > 0.f ? (m_run[nb] + __log2f(lsum)) * 0.69314718055994531f : -INFINITY;
      const int rr = WROWS * wave + 16 * nb + n;  // row within the tile
      const int row = row_lo + rr;
      if (slot < 0) {
        const int tok = q0 + row / g;
        const int qhd = h * g + row % g;
        const int64_t ob = int64_t(tok) * a.o_st + int64_t(qhd) * a.o_sh + 4 * j;
        if (j == 0) a.lse[int64_t(tok) * a.lse_st + qhd] = lse;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const f32x4 o = acc[nb][db] * inv;
          if (a.out_bf16) {
            const uint2 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            *reinterpret_cast<uint2*>(static_cast<__bf16*>(a.out) + ob + 16 * db) = pk;
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ob + 16 * db) = o;
          }
        }
      } else {
        float* po = a.part_o + (int64_t(slot) * ROWS + rr) * D + 4 * j;
        if (j == 0) a.part_lse[int64_t(slot) * ROWS + rr] = lse;
#pragma unroll
        for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4*>(po + 16 * db) = acc[nb][db] * inv;
      }
    }
    if (slot >= 0 && a.fused_merge) finish_split_chunk<D>(a, slot, tid, kPreThreads, &s_last);
  }
}

hipError_t launch_prefill(int head_dim, bool dense, int tile_q, const AttnArgs& a, int grid, hipStream_t stream) {
#define BSK_PRE(D, DN, NB)                                                                         \
  if (head_dim == D && dense == DN && tile_q == 64 * NB) {                                         \
    hipLaunchKernelGGL((prefill_kernel<D, DN, NB>), dim3(grid), dim3(kPreThreads), 0, stream, a); \
    return hipGetLastError();                                                                      \
  }
  BSK_PRE(128, false, 2)
  BSK_PRE(128, true, 2)
  BSK_PRE(64, false, 2)
  BSK_PRE(64, true, 2)
  BSK_PRE(128, false, 4)
  BSK_PRE(128, true, 4)
  BSK_PRE(64, false, 4)
  BSK_PRE(64, true, 4)
#undef BSK_PRE
  return hipErrorInvalidValue;
}

const void* prefill_kernel_ptr(int head_dim, bool dense, int tile_q) {
#define BSK_PRE_PTR(D, DN, NB) \
  if (head_dim == D && dense == DN && tile_q == 64 * NB) return reinterpret_cast<const void*>(&prefill_kernel<D, DN, NB>);
  BSK_PRE_PTR(128, false, 2)
  BSK_PRE_PTR(128, true, 2)
  BSK_PRE_PTR(64, false, 2)
  BSK_PRE_PTR(64, true, 2)
  BSK_PRE_PTR(128, false, 4)
  BSK_PRE_PTR(128, true, 4)
  BSK_PRE_PTR(64, false, 4)
  BSK_PRE_PTR(64, true, 4)
#undef BSK_PRE_PTR
  return nullptr;
}

int prefill_threads() { return kPreThreads; }

}  // namespace bsk
