// 256-row work item with two waves per SIMD in alternating phases: the body of the 256-row
// persistent attention kernel.
//
// Computes what the large-tile item computes (ragged causal prefill, prefill appended after
// cached KV and the composable format's dense shared prefix: FlashInfer 0.6 wiki, "Kernel
// types"; FlashInfer paper summary, "Research methodology" 1), with a different schedule.
//
// On this hardware a SIMD overlaps the matrix-core work of one wave with the vector work of
// another wave well, but one wave's own MFMA and VALU instructions barely overlap.  The item
// therefore runs eight waves (32 query rows each, two 16-row MFMA column blocks) in two groups:
// waves 0-3 and 4-7, one wave of each group per SIMD.  Each wave alternates
//   a matrix phase: O^T += V^T P^T for the previous key tile, then S^T = K Q^T for this one;
//   a vector phase: masks, online softmax (base 2, fp32, lazily moved reference), P in bf16;
// and the second group runs one phase behind the first, so that while one wave of a SIMD is in
// its matrix phase the other is in its vector phase.  Every phase ends with a workgroup barrier
// that keeps the groups in step; both groups pass the same number of barriers (the second
// group idles in the first phase, the first group in the last one).
//
// K and V tiles (64 keys) go through LDS by direct global-to-LDS transfers, double-buffered per
// tensor: at the start of phase 2u the transfers of K tile u+1 and V tile u are issued, and
// they are waited for at the end of phase 2u+1; K tile u is read in phases 2u and 2u+1, V tile
// u in phases 2u+2 and 2u+3, so a buffer is refilled only after the barrier that ends its last
// read.  Swizzles, transposing V reads and the MFMA operand layouts are the large-tile item's.

#pragma once

#include "prefill_item.h"

namespace bsk {

constexpr int kPPWaves = 8;
constexpr int kPPThreads = kPPWaves * kWave;
constexpr int kPPRows = kPPWaves * 32;
constexpr int kNegInfBits = int(0xff800000u);

// LDS of one workgroup: the K and V tiles as in the large-tile item, plus the item's query rows
// (each wave's 32 rows, 16-byte chunks swizzled like the K rows).
template <int D>
struct PrefillPPSmem {
  PrefillSmem<D> kv;
  unsigned short q[kPPRows * D];
};

template <int D, bool DENSE, bool SAME>
__device__ __forceinline__ void prefill_pp_item(const AttnArgs& a, const int32_t* __restrict__ rec,
                                                PrefillPPSmem<D>& smq, int32_t* s_pages, int* s_last) {
  PrefillSmem<D>& sm = smq.kv;
  constexpr int NB = 2;                      // 16-row column blocks per wave
  constexpr int WROWS = 16 * NB;             // rows per wave
  constexpr int ROWS = kPPWaves * WROWS;     // rows per item (the plan's tile_q)
  constexpr int NDB = D / 16;                // 16-column blocks of the output
  constexpr int NKS = D / 32;                // k-steps over d for the logits
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int RPW = kWave / CH;            // key rows one wave-wide transfer fills (1 KB)
  constexpr int NP = kPreKeys / (kPPWaves * RPW);  // transfers per wave per tile and tensor
  constexpr int TILE = kPreKeys * D;         // bf16 per LDS tile
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(NP >= 1, "transfers per wave");
  static_assert(ROWS == kPPRows, "rows per item");

  unsigned short* s_k = sm.k;
  unsigned short* s_v = sm.v;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int grp = wave_u >> 2;  // 0: waves 0-3, 1: waves 4-7 (one phase behind)
  const int n = lane & 15;
  const int j = lane >> 4;

  const __bf16* __restrict__ Qp = static_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ Kp = static_cast<const __bf16*>(a.k);
  const __bf16* __restrict__ Vp = static_cast<const __bf16*>(a.v);
  const int g = a.group;
  const int pmask = (1 << a.page_shift) - 1;
  const uint32_t k_page_bytes = uint32_t(a.k_sp) * 2u;  // the host checks that they fit 32 bits
  const uint32_t v_page_bytes = uint32_t(a.v_sp) * 2u;
  const uint32_t lds_k = lds_addr(s_k), lds_v = lds_addr(s_v);

  // Transfer p of this wave fills tile rows (p * 8 + wave) * RPW .. + RPW - 1; lane l carries
  // physical chunk l % CH of row (p * 8 + wave) * RPW + l / CH.
  int trow[NP], ck[NP], cv[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    trow[p] = (p * kPPWaves + wave) * RPW + lane / CH;
    ck[p] = (lane % CH) ^ swz_k<D>(trow[p]);
    cv[p] = (lane % CH) ^ swz_v<D>(trow[p]);
  }
  const int k_rd = n * D;
  const int k_sw = swz_k<D>(n);
  const int v_row = 4 * j + (n >> 2);
  const int v_sw = swz_v<D>(v_row);
  const int v_half = 4 * (n & 1);

  const int h = rec[IT_H];
  const int row_lo = rec[IT_ROW_LO], row_hi = rec[IT_ROW_HI];
  const int kv_lo = rec[IT_KV_LO], kv_hi = rec[IT_KV_HI];
  const int slot = rec[IT_SLOT];
  const int q0 = rec[IT_Q0];
  const int qlen = rec[IT_QLEN];
  const int L = rec[IT_KVLEN];
  const int kbase = rec[IT_KBASE];

  __syncthreads();  // the previous item is done with the page list and the tiles
  if constexpr (!DENSE) stage_pages(s_pages, a.page_indices, kbase, kv_lo, kv_hi, a.page_shift, tid, kPPThreads);
  __syncthreads();

  // This wave's query rows go to LDS by direct transfers (RPW rows per transfer); rows past the
  // item repeat its last row, whose results are never written.
  int qpos[NB];
  bool row_ok[NB];
  const unsigned short* sq = smq.q + WROWS * wave_u * D;
  {
    const uint32_t lq = lds_addr(smq.q) + uint32_t(WROWS * wave_u * D * 2);
#pragma unroll
    for (int p = 0; p < WROWS / RPW; ++p) {
      const int lr = p * RPW + lane / CH;  // row within the wave's block
      const int row = min(row_lo + WROWS * wave + lr, row_hi - 1);
      const int qi = row / g, qu = row % g;
      const __bf16* src = Qp + int64_t(q0 + qi) * a.q_st + int64_t(h * g + qu) * a.q_sh +
                          8 * ((lane % CH) ^ swz_k<D>(lr));
      dma16(src, lq + uint32_t(p * 1024));
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = row_lo + WROWS * wave + 16 * nb + n;
    row_ok[nb] = row < row_hi;
    qpos[nb] = L - qlen + (row_ok[nb] ? row / g : 0);
  }
  const int wrow0 = row_lo + WROWS * wave_u;
  const int wrow1 = min(row_hi, wrow0 + WROWS) - 1;
  const int wq_lo = __builtin_amdgcn_readfirstlane(L - qlen + (wrow0 < row_hi ? wrow0 / g : 0));
  const int wq_hi = __builtin_amdgcn_readfirstlane(L - qlen + (wrow1 >= wrow0 ? wrow1 / g : 0));
  const bool wave_has_rows = wrow0 < row_hi;
  const bool all_rows = wrow0 + WROWS <= row_hi;

  float m_run[NB], l_run[NB], neg_m[NB], thr[NB];
  f32x4 acc[NB][NDB];  // acc[nb][db][i] = O^T[16 db + 4 j + i][row n of block nb]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
    neg_m[nb] = 0.f;
    thr[nb] = -INFINITY;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[nb][db] = f32x4{0, 0, 0, 0};
  }
  const float inv_scale_log2 = 1.f / a.scale_log2;

  // transfer addressing, as in the large-tile item
  const bool fast_item = DENSE || (kv_lo & (kPreKeys - 1)) == 0;
  const char* kfix[NP];
  const char* vfix[NP];
  int64_t vdel[NP];
  int pslot[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int tok = DENSE ? trow[p] : (trow[p] & pmask);
    const uint32_t koff = uint32_t(2 * (int64_t(h) * a.k_sh + int64_t(tok) * a.k_st) + 16 * ck[p]);
    const uint32_t voff = SAME ? koff - 16 * ck[p] + 16 * cv[p]
                               : uint32_t(2 * (int64_t(h) * a.v_sh + int64_t(tok) * a.v_st) + 16 * cv[p]);
    kfix[p] = reinterpret_cast<const char*>(Kp) + koff;
    vfix[p] = reinterpret_cast<const char*>(Vp) + voff;
    vdel[p] = vfix[p] - kfix[p];
    pslot[p] = trow[p] >> a.page_shift;
  }
  const int p0 = kv_lo >> a.page_shift;

  // Transfers of tile `tile` of one tensor (K if IS_K, else V) into LDS buffer `buf`.
  auto load = [&](int tile, int buf, auto is_k_c) {
    constexpr bool IS_K = decltype(is_k_c)::value;
    const int kt = kv_lo + tile * kPreKeys;
    const uint32_t l0 = (IS_K ? lds_k : lds_v) + uint32_t(buf * TILE * 2);
    const char* base = reinterpret_cast<const char*>(IS_K ? static_cast<const void*>(Kp) : static_cast<const void*>(Vp));
    if (fast_item && kt + kPreKeys <= kv_hi) {
      if constexpr (DENSE) {
        const int64_t tk = 2 * (int64_t(kbase + kt) * (IS_K ? a.k_st : a.v_st));
#pragma unroll
        for (int p = 0; p < NP; ++p)
          dma16((IS_K ? kfix[p] : vfix[p]) + tk, l0 + uint32_t((p * kPPWaves + wave_u) * 1024));
      } else {
        const int sb = (kt >> a.page_shift) - p0;
        uint32_t page[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) page[p] = uint32_t(s_pages[sb + pslot[p]]);
        const int64_t in_page = a.page_shift > 6 ? 2 * (int64_t(kt & pmask) * (IS_K ? a.k_st : a.v_st)) : 0;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const char* src;
          if (IS_K || SAME)
            src = kfix[p] + uint64_t(page[p]) * k_page_bytes + in_page + (IS_K ? 0 : vdel[p]);
          else
            src = vfix[p] + uint64_t(page[p]) * v_page_bytes + in_page;
          dma16(src, l0 + uint32_t((p * kPPWaves + wave_u) * 1024));
        }
      }
    } else {
      // ragged tail or unaligned start: rows past the range repeat the last key (masked later)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int t = min(kt + trow[p], kv_hi - 1);
        const int64_t off =
            IS_K ? kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.k_sp, a.k_sh, a.k_st)
                 : kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.v_sp, a.v_sh, a.v_st);
        dma16(base + 2 * off + 16 * (IS_K ? ck[p] : cv[p]), l0 + uint32_t((p * kPPWaves + wave_u) * 1024));
      }
    }
  };

  const int ntiles = (kv_hi - kv_lo + kPreKeys - 1) / kPreKeys;  // items are never empty
  int clean_hi = all_rows ? kv_hi - kPreKeys : INT_MIN;
  if (a.causal) clean_hi = min(clean_hi, wq_lo - (kPreKeys - 1));
  const int clean_lo = a.window > 0 ? wq_hi - a.window + 1 : INT_MIN;
  clean_hi = __builtin_amdgcn_readfirstlane(clean_hi);

  f32x4 st[2][2][NB];   // logits of the wave's current tile: [32-key half][16-key block][row block]
  bf16x8 pb[2][NB];     // probabilities of the wave's previous tile, MFMA B operands per half
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      st[x][0][nb] = f32x4{0, 0, 0, 0};
      st[x][1][nb] = f32x4{0, 0, 0, 0};
      pb[x][nb] = bf16x8{};
    }

  // Matrix phase for tile t: PV of tile t - 1 (V buffer VB), then the logits of tile t (K
  // buffer KB).  Operands are staged a few fragments at a time: four V^T fragments, then the K
  // fragments of one 32-wide d step for all four 16-key blocks.
  auto matrix_phase = [&](int t, auto kb_c, auto vb_c) {
    constexpr int KB = decltype(kb_c)::value;
    constexpr int VBUF = decltype(vb_c)::value;
    if (t >= 1) {
      const unsigned short* sv = s_v + VBUF * TILE;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const unsigned short* vb = sv + (32 * ks + v_row) * D + v_half;
#pragma unroll
        for (int d0 = 0; d0 < NDB; d0 += 4) {
          bf16x8 va[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int off = 8 * ((2 * (d0 + i) + ((n & 3) >> 1)) ^ v_sw);
            va[i] = ds_read_tr_pair(vb + off, vb + off + 16 * D);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              acc[nb][d0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[i], pb[ks][nb], acc[nb][d0 + i], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (t < ntiles) {
      const unsigned short* sk = s_k + KB * TILE;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mh = 0; mh < 2; ++mh)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) st[ks][mh][nb] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        bf16x8 qf[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          qf[nb] = *reinterpret_cast<const bf16x8*>(sq + (16 * nb + n) * D + 8 * ((4 * s + j) ^ k_sw));
        bf16x8 kf[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int mh = 0; mh < 2; ++mh)
            kf[ks][mh] = *reinterpret_cast<const bf16x8*>(sk + 16 * (2 * ks + mh) * D + k_rd + 8 * ((4 * s + j) ^ k_sw));
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int mh = 0; mh < 2; ++mh)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              st[ks][mh][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks][mh], qf[nb], st[ks][mh][nb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Vector phase for tile t: masks, online softmax, P.
  auto vector_phase = [&](int t) {
    const int kt = kv_lo + t * kPreKeys;
    if (!(kt >= clean_lo && kt <= clean_hi)) {
      // Masks in vector registers only: key t is visible iff t < hi and (t >= lo or t < sk), i.e.
      // iff min(hi - 1 - t, max(t - lo, sk - 1 - t)) >= 0; its sign selects -inf.  The per-tile
      // terms pass through empty asm statements so that the compiler neither folds the sixteen
      // key offsets into them nor keeps the results in registers across the loop.
      const int tb = kt + 4 * j;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int hi = row_ok[nb] ? (a.causal ? min(kv_hi, qpos[nb] + 1) : kv_hi) : -(1 << 30);
        int e1 = hi - 1 - tb;
        asm volatile("" : "+v"(e1));
        if (a.window > 0) {
          int e2 = tb - (qpos[nb] - a.window + 1);
          int e3 = a.sink - 1 - tb;
          asm volatile("" : "+v"(e2), "+v"(e3));
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int mh = 0; mh < 2; ++mh)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int c = 16 * (2 * ks + mh) + i;
                const int m = min(e1 - c, max(e2 + c, e3 - c)) >> 31;
                st[ks][mh][nb][i] = __int_as_float((m & kNegInfBits) | (~m & __float_as_int(st[ks][mh][nb][i])));
              }
        } else {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int mh = 0; mh < 2; ++mh)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int m = (e1 - (16 * (2 * ks + mh) + i)) >> 31;
                st[ks][mh][nb][i] = __int_as_float((m & kNegInfBits) | (~m & __float_as_int(st[ks][mh][nb][i])));
              }
        }
      }
    }
    float lmax[NB];
    uint64_t grow = 0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float x = fmaxf(fmaxf(st[0][0][nb][0], st[0][0][nb][1]), st[0][0][nb][2]);
      x = fmaxf(fmaxf(x, st[0][0][nb][3]), st[0][1][nb][0]);
      x = fmaxf(fmaxf(x, st[0][1][nb][1]), st[0][1][nb][2]);
      x = fmaxf(fmaxf(x, st[0][1][nb][3]), st[1][0][nb][0]);
      x = fmaxf(fmaxf(x, st[1][0][nb][1]), st[1][0][nb][2]);
      x = fmaxf(fmaxf(x, st[1][0][nb][3]), st[1][1][nb][0]);
      x = fmaxf(fmaxf(x, st[1][1][nb][1]), st[1][1][nb][2]);
      lmax[nb] = fmaxf(x, st[1][1][nb][3]);
      grow |= __builtin_amdgcn_ballot_w64(lmax[nb] > thr[nb]);
    }
    if (grow) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float bm = wave_max_xor16_32(lmax[nb]) * a.scale_log2;  // scale > 0 keeps the max
        if (bm > m_run[nb] + kPreRescaleSlack) {
          const float alpha = m_run[nb] == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[nb] - bm);
          l_run[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc[nb][db] *= alpha;
          m_run[nb] = bm;
          neg_m[nb] = -bm;
          thr[nb] = (bm + kPreRescaleSlack) * inv_scale_log2;
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        u32x4 pw;
        float pr[2][4];
#pragma unroll
        for (int mh = 0; mh < 2; ++mh) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pr[mh][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[ks][mh][nb][i], a.scale_log2, neg_m[nb]));
          // MFMA k elements 0..3 hold key block 2ks, elements 4..7 block 2ks+1
          pw[2 * mh] = pack_bf16x2(pr[mh][0], pr[mh][1]);
          pw[2 * mh + 1] = pack_bf16x2(pr[mh][2], pr[mh][3]);
        }
        pb[ks][nb] = __builtin_bit_cast(bf16x8, pw);
        l_run[nb] += ((pr[0][0] + pr[0][1]) + (pr[0][2] + pr[0][3])) + ((pr[1][0] + pr[1][1]) + (pr[1][2] + pr[1][3]));
      }
  };

  // K tile 0 (and the query rows) before the first phase
  load(0, 0, Const<bool, true>{});
  wait_dma();
  __syncthreads();

  // Global phase p: the first group's matrix phase of tile t is phase 2t and its vector phase
  // 2t + 1; the second group's are 2t + 1 and 2t + 2.  At the start of an even phase 2u the
  // waves in it issue their transfers of K tile u + 1 and V tile u; at the end of an odd phase
  // they wait for them.  Every wave passes 2 ntiles + 2 barriers.
  auto issue = [&](int u) {
    if (u + 1 < ntiles) load(u + 1, (u + 1) & 1, Const<bool, true>{});
    if (u < ntiles) load(u, u & 1, Const<bool, false>{});
  };
  auto end_phase = [&](bool wait) {
    if (wait) wait_dma();
    __syncthreads();
  };
  // Matrix phase of tile t, then (t < ntiles) its vector phase; PAR = t & 1 selects the K buffer
  // of tile t and the V buffer of tile t - 1 at compile time.  Returns false after the last one.
  auto step = [&](int t, auto par_c) {
    constexpr int PAR = decltype(par_c)::value;
    if (grp == 0) issue(t);
    if (wave_has_rows) matrix_phase(t, Const<int, PAR>{}, Const<int, PAR ^ 1>{});
    end_phase(grp == 1);
    if (t == ntiles) return false;
    if (grp == 1) issue(t + 1);
    if (wave_has_rows) vector_phase(t);
    end_phase(grp == 0);
    return true;
  };
  if (grp == 1) {  // the second group's idle first phase
    issue(0);
    end_phase(false);
  }
  for (int t = 0;; t += 2) {
    if (!step(t, Const<int, 0>{})) break;
    if (!step(t + 1, Const<int, 1>{})) break;
  }
  if (grp == 0) end_phase(true);  // the first group's idle last phase

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
      if (j == 0) store_part(a.part_lse + int64_t(slot) * ROWS + rr, lse, a.fused_merge);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
          const f32x4 v = acc[nb][db] * inv;
          store_part4(po + 16 * db, v[0], v[1], v[2], v[3], a.fused_merge);
        }
    }
  }
  if (slot >= 0 && a.fused_merge) finish_split_chunk<D>(a, slot, tid, kPPThreads, s_last);
}

}  // namespace bsk
