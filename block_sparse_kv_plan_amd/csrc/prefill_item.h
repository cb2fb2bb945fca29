// Large-tile work item (128 or 256 query rows): the body of the large-tile
// persistent attention kernel, shared with the mixed launch.
//
// Serves ragged causal prefill, including prefill appended after cached KV
// (FlashInfer 0.6 wiki, "Kernel types": Prefill, compute-bound, chunked
// prefill) and the dense shared prefix of the composable format (FlashInfer
// paper summary, "Research methodology" 1), where all branch queries of a
// kv head form one tile and read the prefix once.  Same persistent
// plan-driven structure as the small-tile kernel; bf16 only.
//
// Per item (request r, kv head h, rows [row_lo, row_lo + 16 NB WAVES), keys
// [kv_lo, kv_hi)): each of the WAVES waves owns 16 NB rows (NB 16-row MFMA
// column blocks) and the whole key range.  Keys go through LDS in 64-key
// tiles, double-buffered, loaded by direct global-to-LDS transfers
// (global_load_lds_dwordx4: every lane moves 16 bytes, a wave fills 1 KB
// of LDS, no registers involved); the next tile's transfers are issued right
// after the barrier that opens the current tile, so one barrier per tile
// suffices.  LDS rows are unpadded; their 16-byte chunks are XOR-swizzled
// by row so that both read patterns below are free of bank conflicts.
//   S^T (64 x 16 NB) = K Q^T    16x16x32 bf16 MFMA, K from LDS, q in registers
//   online softmax in base 2, fp32; masks are evaluated only on tiles that
//   cross a boundary (range end, causal diagonal, window); the accumulator
//   is rescaled only when a row's max grows by more than 2^8
//   O^T (D x 16 NB) += V^T P^T  16x16x32 bf16 MFMA; V^T comes from
//   transposing LDS reads, the MFMA key index being mapped to the keys
//   whose probabilities the lane already holds
// and every wave writes its own rows (output or partial state).
//
// Every K/V tile read from LDS is shared by all NB row blocks of a wave and by
// all WAVES waves of the workgroup.  The kernels use NB = 2 (32 rows per wave)
// with four waves (128-row items, two workgroups per CU) or eight waves
// (256-row items, one workgroup per CU); either way a SIMD runs two waves, so
// one's MFMAs overlap the other's softmax.  NB = 4 (64 rows per wave, one wave
// per SIMD) halves the LDS reads per MFMA but loses that overlap and was slower.
//
// The logit max uses fmaxf on values that are never NaN (masked logits are
// replaced by -inf before it), so the files that include this one are built
// without NaN semantics and the max needs no operand canonicalisation.

#pragma once

#include "device.h"

namespace bsk {

constexpr int kPreWaves = 4;
constexpr int kPreThreads = kPreWaves * kWave;
constexpr int kPreKeys = 64;                  // keys per LDS tile
constexpr float kPreRescaleSlack = 8.f;       // log2 units

// XOR swizzles of the 16-byte chunks of an LDS row.  K rows are read by 16 lanes at a time,
// rows n = 0..15 at one logical chunk; V rows by the transposing reads, 4 rows x 2 chunks x 2
// halves per 16 lanes and two such groups at a time.  Both patterns hit distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? ((2 * (r & 3)) ^ (8 * ((r >> 2) & 1))) : (2 * ((r >> 1) & 3));
}

// A compile-time value passed to a generic lambda.
template <typename T, T V>
struct Const {
  static constexpr T value = V;
};

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

// LDS of one workgroup for a large-tile item: double-buffered K and V tiles of kPreKeys rows,
// unpadded (the 16-byte chunks are swizzled instead).  The variable holding it is aligned to
// 1 KB so that the swizzles see the bank layout they were chosen for.
template <int D>
struct PrefillSmem {
  static constexpr int TILE = kPreKeys * D;
  unsigned short k[2 * TILE];
  unsigned short v[2 * TILE];
};

// SAME: K and V share page/head/token strides; a V address is the K address plus the K-to-V
// pointer distance.
// SUM_MFMA: the bf16 probability sum (below) comes from one more MFMA per half against a ones
// operand, else from v_dot2 instructions (fewer registers: the mixed launch's budget is full).
template <int D, bool DENSE, int NB, bool SAME, int WAVES = kPreWaves, bool SUM_MFMA = true>
__device__ __forceinline__ void prefill_item(const AttnArgs& a, const int32_t* __restrict__ rec, PrefillSmem<D>& sm,
                                             int32_t* s_pages, int* s_last) {
  constexpr int ROWS = WAVES * 16 * NB;      // query rows per item (the plan's tile_q)
  constexpr int WROWS = 16 * NB;             // rows per wave
  constexpr int NDB = D / 16;                // 16-column blocks of the output
  constexpr int NKS = D / 32;                // k-steps over d for the logits
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int RPW = kWave / CH;            // key rows one wave-wide transfer fills (1 KB)
  constexpr int NP = kPreKeys / (WAVES * RPW);  // transfers per wave per tile and tensor
  constexpr int NTHREADS = WAVES * kWave;
  constexpr int TILE = kPreKeys * D;         // bf16 per LDS tile
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(NB == 2 || NB == 4, "row blocks per wave");
  static_assert(TILE == PrefillSmem<D>::TILE, "tile size");

  unsigned short* s_k = sm.k;
  unsigned short* s_v = sm.v;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int n = lane & 15;
  const int j = lane >> 4;

  const __bf16* __restrict__ Qp = static_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ Kp = static_cast<const __bf16*>(a.k);
  const __bf16* __restrict__ Vp = static_cast<const __bf16*>(a.v);
  const int g = a.group;
  const int pmask = (1 << a.page_shift) - 1;
  // page strides in bytes; the host checks that they fit 32 bits
  const uint32_t k_page_bytes = uint32_t(a.k_sp) * 2u;
  const uint32_t v_page_bytes = uint32_t(a.v_sp) * 2u;
  const uint32_t lds_k = lds_addr(s_k), lds_v = lds_addr(s_v);

  // Transfer p of this wave fills tile rows (p * 4 + wave) * RPW .. + RPW - 1; lane l carries
  // physical chunk l % CH of row (p * 4 + wave) * RPW + l / CH, i.e. the logical chunk that the
  // row's swizzle maps there.
  int trow[NP], ck[NP], cv[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    trow[p] = (p * WAVES + wave) * RPW + lane / CH;
    ck[p] = (lane % CH) ^ swz_k<D>(trow[p]);
    cv[p] = (lane % CH) ^ swz_v<D>(trow[p]);
  }
  // LDS read offsets (elements) that do not change from tile to tile
  const int k_rd = n * D + 8 * 0;  // row n of each 16-key block; chunk added per k-step
  const int k_sw = swz_k<D>(n);    // swizzle of rows 16 mb + n
  const int v_row = 4 * j + (n >> 2);
  const int v_sw = swz_v<D>(v_row);  // same for rows v_row + 16 i
  const int v_half = 4 * (n & 1);

  {
    const int r = rec[IT_R], h = rec[IT_H];
    const int row_lo = rec[IT_ROW_LO], row_hi = rec[IT_ROW_HI];
    const int kv_lo = rec[IT_KV_LO], kv_hi = rec[IT_KV_HI];
    const int slot = rec[IT_SLOT];
    const int q0 = rec[IT_Q0];
    const int qlen = rec[IT_QLEN];
    const int L = rec[IT_KVLEN];
    const int kbase = rec[IT_KBASE];
    (void)r;

    __syncthreads();  // the previous item is done with the page list and the tiles
    if constexpr (!DENSE) stage_pages(s_pages, a.page_indices, kbase, kv_lo, kv_hi, a.page_shift, tid, NTHREADS);
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
    const int wrow0 = row_lo + WROWS * wave_u;  // wave-uniform: the tile tests below stay scalar
    const int wrow1 = min(row_hi, wrow0 + WROWS) - 1;  // may be < wrow0 for an empty wave
    const int wq_lo = __builtin_amdgcn_readfirstlane(L - qlen + (wrow0 < row_hi ? wrow0 / g : 0));
    const int wq_hi = __builtin_amdgcn_readfirstlane(L - qlen + (wrow1 >= wrow0 ? wrow1 / g : 0));
    const bool wave_has_rows = wrow0 < row_hi;
    const bool all_rows = wrow0 + WROWS <= row_hi;

    // l_run: fp32 sum of the probabilities (the LSE).  lb: the same probabilities as the bf16 PV
    // operand holds them, which normalises O, so that a key that dominates a row contributes its V
    // row exactly instead of with its probability's bf16 rounding (up to 2^-9 of the row).  With
    // SUM_MFMA every element of lb_acc[nb] ends up holding the row's sum; otherwise lb_run[nb]
    // holds this lane's share.
    float m_run[NB], l_run[NB], lb_run[NB];
    f32x4 lb_acc[NB];
    f32x4 acc[NB][NDB];  // acc[nb][db][i] = O^T[16 db + 4 j + i][row n of block nb]
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = -INFINITY;
      l_run[nb] = 0.f;
      lb_run[nb] = 0.f;
      lb_acc[nb] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[nb][db] = f32x4{0, 0, 0, 0};
    }

    // Transfer addressing.  When tiles start at multiples of 64 keys (always for dense KV; for
    // paged KV when the item does), a full tile's row t sits in page slot (kt >> shift) - p0 +
    // (t >> shift) at in-page token (kt & pmask) + (t & pmask): a page of <= 64 keys divides the
    // tile (the in-page part of kt is zero), a larger page holds all of it.  The 32-bit per-row
    // part (head, in-page or in-tile token, chunk) is below the page stride (paged) or 2^31
    // (dense, checked by the host).  kfix[p] / vfix[p] are the K / V addresses of transfer p's
    // row in page 0 (paged) or at key 0 (dense); with shared strides the V address is the K
    // address plus vdel[p].
    const bool fast_item = DENSE || (kv_lo & (kPreKeys - 1)) == 0;
    const char* kfix[NP];
    const char* vfix[NP];
    int64_t vdel[NP];
    int pslot[NP];  // page slot of transfer p's row, relative to the tile's first slot
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

    auto load_tile = [&](int kt, int buf) {
      const uint32_t lk0 = lds_k + uint32_t(buf * TILE * 2), lv0 = lds_v + uint32_t(buf * TILE * 2);
      if (fast_item && kt + kPreKeys <= kv_hi) {
        if constexpr (DENSE) {
          const int64_t tk = 2 * (int64_t(kbase + kt) * a.k_st);
          const int64_t tv = 2 * (int64_t(kbase + kt) * a.v_st);
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const uint32_t lo = uint32_t((p * WAVES + wave_u) * 1024);
            const char* ka = kfix[p] + tk;
            dma16(ka, lk0 + lo);
            dma16(SAME ? ka + vdel[p] : vfix[p] + tv, lv0 + lo);
          }
        } else {
          // All page ids first: the transfers are ordered memory operations, so an LDS read
          // placed after one of them would wait on its own.
          const int sb = (kt >> a.page_shift) - p0;
          uint32_t page[NP];
#pragma unroll
          for (int p = 0; p < NP; ++p) page[p] = uint32_t(s_pages[sb + pslot[p]]);
          // pages of more than 64 keys: the tile starts inside the page
          auto issue = [&](auto big_c) {
            constexpr bool BIG = decltype(big_c)::value;
            const int64_t tk = BIG ? 2 * (int64_t(kt & pmask) * a.k_st) : 0;
            const int64_t tv = BIG ? 2 * (int64_t(kt & pmask) * a.v_st) : 0;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              const uint32_t lo = uint32_t((p * WAVES + wave_u) * 1024);
              const char* ka = kfix[p] + uint64_t(page[p]) * k_page_bytes;
              if constexpr (BIG) ka += tk;
              dma16(ka, lk0 + lo);
              if constexpr (SAME) {
                dma16(ka + vdel[p], lv0 + lo);
              } else {
                const char* va = vfix[p] + uint64_t(page[p]) * v_page_bytes;
                if constexpr (BIG) va += tv;
                dma16(va, lv0 + lo);
              }
            }
          };
          if (a.page_shift > 6)
            issue(Const<bool, true>{});
          else
            issue(Const<bool, false>{});
        }
      } else {
        // ragged tail or unaligned start: rows past the range repeat the last key (masked later)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int t = min(kt + trow[p], kv_hi - 1);
          const int64_t ko = kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.k_sp, a.k_sh, a.k_st);
          const int64_t vo =
              SAME ? ko : kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.v_sp, a.v_sh, a.v_st);
          const uint32_t lo = uint32_t((p * WAVES + wave_u) * 1024);
          dma16(Kp + ko + 8 * ck[p], lk0 + lo);
          dma16(Vp + vo + 8 * cv[p], lv0 + lo);
        }
      }
    };

    const int ntiles = (kv_hi - kv_lo + kPreKeys - 1) / kPreKeys;  // items are never empty
    // A tile starting at key kt needs no mask for any row of this wave iff clean_lo <= kt <=
    // clean_hi: the wave's rows are all in the item, the tile ends inside the key range and at
    // or before the wave's first query position (causal), and every key of it is inside the
    // window of the wave's last query position.
    int clean_hi = all_rows ? kv_hi - kPreKeys : INT_MIN;
    if (a.causal) clean_hi = min(clean_hi, wq_lo - (kPreKeys - 1));
    const int clean_lo = a.window > 0 ? wq_hi - a.window + 1 : INT_MIN;
    clean_hi = __builtin_amdgcn_readfirstlane(clean_hi);

    // Per row block besides m_run and l_run: the exponent offset (-m_run, or 0 before any
    // visible key) and the raw logit above which the reference has to move.
    const float inv_scale_log2 = 1.f / a.scale_log2;
    float neg_m[NB], thr[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      neg_m[nb] = 0.f;
      thr[nb] = -INFINITY;
    }

    // One 64-key tile from LDS buffer BUF, a compile-time constant so that every LDS read
    // address is a per-lane constant plus an immediate offset.
    auto tile_step = [&](int tile, auto buf_c) {
      constexpr int BUF = decltype(buf_c)::value;
      const int kt = kv_lo + tile * kPreKeys;
      wait_dma();        // this wave's transfers of the tile have landed
      __syncthreads();   // ... and every other wave's; the other buffer is free again
      if (tile + 1 < ntiles) load_tile(kt + kPreKeys, BUF ^ 1);  // in flight during this tile's math
      if (!wave_has_rows) return;
      const unsigned short* sk = s_k + BUF * TILE;
      const unsigned short* sv = s_v + BUF * TILE;

      // masks only where the tile crosses a boundary for some row of this wave
      const bool clean = kt >= clean_lo && kt <= clean_hi;
      // Logits of a 32-key half: all its K fragments are read first (their LDS latencies
      // overlap), then the MFMAs.
      auto logits = [&](int ks, f32x4 (&st)[2][NB]) {
#pragma unroll
        for (int mh = 0; mh < 2; ++mh)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) st[mh][nb] = f32x4{0, 0, 0, 0};
        bf16x8 kf[2][NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s)
#pragma unroll
          for (int mh = 0; mh < 2; ++mh)
            kf[mh][s] = *reinterpret_cast<const bf16x8*>(sk + 16 * (2 * ks + mh) * D + k_rd + 8 * ((4 * s + j) ^ k_sw));
#pragma unroll
        for (int s = 0; s < NKS; ++s)
#pragma unroll
          for (int mh = 0; mh < 2; ++mh)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              st[mh][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mh][s], qf[nb][s], st[mh][nb], 0, 0, 0);
      };
      // With two row blocks the logits of both halves are issued first: each half's softmax then
      // runs on the VALU while the matrix cores still work on the other half's logits (or the
      // previous PV).  With four row blocks the registers allow only one half at a time.
      constexpr int LIVE = NB <= 2 ? 2 : 1;
      f32x4 st2[LIVE][2][NB];
      if constexpr (LIVE == 2) {
        logits(0, st2[0]);
        logits(1, st2[1]);
      }
      // masks of half ks, only where the tile crosses a boundary for some row of this wave.  The
      // lane's keys are base + 16 mh + i, so without a window a key is visible iff its constant
      // offset is below the row's bound minus base: one compare with an immediate per key.
      auto mask_half = [&](f32x4 (&st)[2][NB], int ks) {
        const int base = kt + 32 * ks + 4 * j;
        if (a.window > 0) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const RowMask rm = row_mask(row_ok[nb], qpos[nb], kv_hi, a.causal, a.window, a.sink);
#pragma unroll
            for (int mh = 0; mh < 2; ++mh)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                st[mh][nb][i] = row_sees(rm, base + 16 * mh + i) ? st[mh][nb][i] : -INFINITY;
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            // keys [.., hi) are visible: the range end and, if causal, the row's position
            const int hi = a.causal ? min(kv_hi, qpos[nb] + 1) : kv_hi;
            const int lim = row_ok[nb] ? hi - base : 0;  // offsets below lim are visible
#pragma unroll
            for (int mh = 0; mh < 2; ++mh)
#pragma unroll
              for (int i = 0; i < 4; ++i) st[mh][nb][i] = 16 * mh + i < lim ? st[mh][nb][i] : -INFINITY;
          }
        }
      };
      auto half_max = [&](const f32x4 (&st)[2][NB], int nb) {
        float x = fmaxf(fmaxf(st[0][nb][0], st[0][nb][1]), st[0][nb][2]);
        x = fmaxf(fmaxf(x, st[0][nb][3]), st[1][nb][0]);
        x = fmaxf(fmaxf(x, st[1][nb][1]), st[1][nb][2]);
        return fmaxf(x, st[1][nb][3]);
      };
      // Online softmax with a lazily moved reference: each lane checks its own logits against
      // the row's threshold; only if some lane exceeds it is the row max reduced across the
      // row's four lanes and the state rescaled.
      auto maybe_rescale = [&](const float (&lmax)[NB]) {
        uint64_t grow = 0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) grow |= __builtin_amdgcn_ballot_w64(lmax[nb] > thr[nb]);
        if (grow) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const float bm = wave_max_xor16_32(lmax[nb]) * a.scale_log2;  // scale > 0 keeps the max
            if (bm > m_run[nb] + kPreRescaleSlack) {
              const float alpha = m_run[nb] == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[nb] - bm);
              l_run[nb] *= alpha;
              if constexpr (SUM_MFMA)
                lb_acc[nb] *= alpha;
              else
                lb_run[nb] *= alpha;
#pragma unroll
              for (int db = 0; db < NDB; ++db) acc[nb][db] *= alpha;
              m_run[nb] = bm;
              neg_m[nb] = -bm;
              thr[nb] = (bm + kPreRescaleSlack) * inv_scale_log2;
            }
          }
        }
      };
      // P of a half (bf16 operand of the PV product) and the row sums
      auto probs = [&](const f32x4 (&st)[2][NB], bf16x8 (&pb)[NB]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          u32x4 pw;
          float pr[2][4];
#pragma unroll
          for (int mh = 0; mh < 2; ++mh) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pr[mh][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[mh][nb][i], a.scale_log2, neg_m[nb]));
            // MFMA k elements 0..3 hold key block 2ks, elements 4..7 block 2ks+1
            pw[2 * mh] = pack_bf16x2(pr[mh][0], pr[mh][1]);
            pw[2 * mh + 1] = pack_bf16x2(pr[mh][2], pr[mh][3]);
          }
          pb[nb] = __builtin_bit_cast(bf16x8, pw);
          // the row sum adds the fp32 values: the log-sum-exp keeps their precision
          l_run[nb] += ((pr[0][0] + pr[0][1]) + (pr[0][2] + pr[0][3])) + ((pr[1][0] + pr[1][1]) + (pr[1][2] + pr[1][3]));
          if constexpr (!SUM_MFMA)
            lb_run[nb] = add_bf16x2(pw[3], add_bf16x2(pw[2], add_bf16x2(pw[1], add_bf16x2(pw[0], lb_run[nb]))));
        }
      };
      // O^T[d][row] += V^T P^T for half ks.  MFMA k index 8j+e <-> key 32ks + 4j + (e&3) + 16(e>>2):
      // the keys whose probabilities this lane holds.  The V^T operand comes from two transposing
      // LDS reads: in each 16-lane group, lane k points at 4 columns of key row k/4 and gets back
      // one column of 4 keys, so lane (n, j) receives V[key(8j+e)][16 db + n].
      auto pv = [&](const bf16x8 (&pb)[NB], int ks) {
        const unsigned short* vb = sv + (32 * ks + v_row) * D + v_half;
        constexpr int VB = NB <= 2 ? NDB : 2;  // V^T operands read ahead of their MFMAs
#pragma unroll
        for (int d0 = 0; d0 < NDB; d0 += VB) {
          bf16x8 va[VB];
#pragma unroll
          for (int i = 0; i < VB; ++i) {
            const int off = 8 * ((2 * (d0 + i) + ((n & 3) >> 1)) ^ v_sw);
            va[i] = ds_read_tr_pair(vb + off, vb + off + 16 * D);
          }
#pragma unroll
          for (int i = 0; i < VB; ++i)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              acc[nb][d0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[i], pb[nb], acc[nb][d0 + i], 0, 0, 0);
        }
        if constexpr (SUM_MFMA) {
          const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            lb_acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[nb], lb_acc[nb], 0, 0, 0);
        }
      };

      if constexpr (LIVE == 2) {
        // Both halves' logits are in registers: the reference moves at most once per tile (from
        // the maximum over both halves), so no branch separates half 1's exponentials from half
        // 0's PV products, and the matrix cores run those products while the exponentials go
        // through the transcendental unit.
        if (!clean) {
          mask_half(st2[0], 0);
          mask_half(st2[1], 1);
        }
        float lmax[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) lmax[nb] = fmaxf(half_max(st2[0], nb), half_max(st2[1], nb));
        maybe_rescale(lmax);
        bf16x8 p0[NB], p1[NB];
        probs(st2[0], p0);
        pv(p0, 0);
        probs(st2[1], p1);
        pv(p1, 1);
      } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          logits(ks, st2[0]);
          f32x4 (&st)[2][NB] = st2[0];
          if (!clean) mask_half(st, ks);
          float lmax[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) lmax[nb] = half_max(st, nb);
          maybe_rescale(lmax);
          bf16x8 pb[NB];
          probs(st, pb);
          pv(pb, ks);
        }
      }
    };

    wait_vm();  // q fragments and page ids are in registers before the tile loop starts
    if (ntiles > 0) load_tile(kv_lo, 0);
    // two tiles per iteration, one from each LDS buffer; every wave passes the same barriers
    for (int tile = 0; tile < ntiles; tile += 2) {
      tile_step(tile, Const<int, 0>{});
      if (tile + 1 < ntiles) tile_step(tile + 1, Const<int, 1>{});
    }

    // epilogue: each lane owns row n of each row block and columns 16 db + 4 j .. + 3
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float lsum = wave_sum_xor16_32(l_run[nb]);
      const float lbsum = SUM_MFMA ? lb_acc[nb][0] : wave_sum_xor16_32(lb_run[nb]);
      if (!row_ok[nb]) continue;
      const float inv = lbsum > 0.f ? 1.f / lbsum : 0.f;
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
    if (slot >= 0 && a.fused_merge) finish_split_chunk<D>(a, slot, tid, NTHREADS, s_last);
  }
}

}  // namespace bsk
