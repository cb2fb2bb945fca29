// Small-tile work item (16 query rows): the body of the small-tile persistent
// attention kernel, shared with the mixed launch.
//
// Serves decode -- query length 1, one row per q head of a GQA group, the
// HBM-bound case of the FlashInfer 0.6 wiki ("Kernel types": Decode) -- and
// short multi-token queries.  One workgroup is one persistent worker: it
// walks its item list from the int workspace (FlashInfer paper summary,
// "Research methodology" 3: the CPU plan cached on the GPU drives a fixed
// launch).  Per item:
//
//   * the item's page ids are staged in LDS (FlashInfer 0.6 wiki,
//     "Architecture" 1: page indices prefetched into shared memory);
//   * keys are walked in 16-key blocks aligned to multiples of 16, so with
//     pages of >= 16 keys a block lies in one page and needs one page id;
//     the four waves take interleaved blocks and keep the next block's
//     loads in flight while consuming the current one;
//   * S^T = K Q^T on MFMA with the 16 keys on the M side and the (up to 16)
//     query rows on the N side: each lane ends up owning one query row, so
//     the row max / sum take two cross-lane steps;
//   * online softmax in base 2 (log2 e folded into the scale); the output
//     accumulator is rescaled only when a row's running max grows by more
//     than 2^8 (values stay exact: numerator and denominator share the max);
//   * O^T += V^T P^T on bf16 MFMA without any LDS transpose: each lane loads
//     whole 16-byte pieces of four V rows (fully coalesced), and the MFMA's
//     key index k = 4j+e is mapped to key 4e+j so that the A operand is a
//     repack of those registers; the K rows are loaded in the matching
//     transposed order (lane row m holds key 4(m%4) + m/4) so the logits
//     land in the lanes that need them as the B operand;
//   * the four waves' states are combined through LDS; a single-chunk item
//     writes O and LSE, a chunk of a split unit writes its partial state.
//
// f32 inputs use the 16x16x4 f32 MFMA (one k element per lane), which
// reads V straight from memory.
//
// Fused RoPE (bf16 cache): q and every key are rotated in fp32 with a cos/sin
// table (the cache holds K unrotated).  Each rotated vector x is split into
// two fp16 vectors, x1 = fp16(x) and x2 = fp16(x - x1), and a logit is
// q1.k1 + q2.k1 + q1.k2: three fp16 MFMAs per k-step, with about 22
// significant bits instead of fp16's 11.  A single fp16 rounding leaves each
// logit an error of about 3e-4 (rms, d = 64 or 128), which a row whose softmax
// one key dominates passes straight into its LSE: over 1e-3 on some rows.
// Rotated values must stay inside fp16's range (|x| < 65504).

#pragma once

#include "device.h"

namespace bsk {

constexpr int kDecRows = 16;
constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr float kRescaleSlack = 8.f;  // log2 units: rescale only when the max grows by > 2^8

enum : int { ROPE_NONE = 0, ROPE_STREAMING = 1, ROPE_ABSOLUTE = 2 };

// Rotate-half RoPE on a lane's fragment pair: lo holds elements k..k+7 of
// the first half, hi the matching k+D/2.. elements; c4 holds the (cos, sin)
// pairs of k..k+7 for the position.
__device__ __forceinline__ void rope8(float* lo, float* hi, const float4* c4) {
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    const float4 t = c4[e2];  // cos_e, sin_e, cos_e+1, sin_e+1
    const int e = 2 * e2;
    float x = lo[e], y = hi[e];
    lo[e] = x * t.x - y * t.y;
    hi[e] = y * t.x + x * t.y;
    x = lo[e + 1];
    y = hi[e + 1];
    lo[e + 1] = x * t.z - y * t.w;
    hi[e + 1] = y * t.z + x * t.w;
  }
}

__device__ __forceinline__ void unpack_bf16x8(const bf16x8& v, float* f) {
  const u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_lo(u[e]);
    f[2 * e + 1] = bf16_hi(u[e]);
  }
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// 8 floats -> fp16x8, rounded to nearest even (four packed conversions)
__device__ __forceinline__ f16x8 to_f16x8(const float* f) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f16x2_t h = __builtin_convertvector((f32x2{f[2 * e], f[2 * e + 1]}), f16x2_t);
    r[2 * e] = h[0];
    r[2 * e + 1] = h[1];
  }
  return r;
}

// What rounding to fp16 left out of 8 floats (h = to_f16x8(f)), itself rounded to fp16.
__device__ __forceinline__ f16x8 f16_residual(const float* f, const f16x8& h) {
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = f[e] - float(h[e]);
  return to_f16x8(r);
}

// Element e of four 8-element pieces (a, b, c, d), as an MFMA k-quad.
__device__ __forceinline__ i16x4 gather_e(const u32x4& a, const u32x4& b, const u32x4& c, const u32x4& d, int e) {
  const int w = e >> 1;
  // v_perm_b32 selector: low halves (bytes 1:0 of each source) or high halves (bytes 3:2)
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
  u32x2 r;
  r[0] = __builtin_amdgcn_perm(b[w], a[w], sel);
  r[1] = __builtin_amdgcn_perm(d[w], c[w], sel);
  return __builtin_bit_cast(i16x4, r);
}

// LDS of one workgroup for a small-tile item: the four waves' accumulators, maxima and sums
// for the combine step (rows padded by 4 floats).
template <int D>
struct DecodeSmem {
  float acc[kDecWaves * 16 * (D + 4)];
  float m[kDecWaves][16];
  float l[kDecWaves][16];
  float lb[kDecWaves][16];
};

// SAME: K and V share page/head/token strides, so one offset serves both tensors.
template <typename T, int D, bool DENSE, int ROPE, bool SAME>
__device__ __forceinline__ void decode_item(const AttnArgs& a, const int32_t* __restrict__ rec, DecodeSmem<D>& sm,
                                            int32_t* s_pages, int* s_last, int part_rows) {
  constexpr bool BF = __is_same(T, __bf16);
  constexpr int NKS = BF ? D / 32 : D / 4;  // MFMA k-steps over d for the logits
  constexpr int NACC = BF ? 8 : D / 16;     // f32x4 accumulators per lane
  constexpr int HALF_KS = D / 64;           // bf16 k-step offset of the rotate-half partner
  constexpr int CHUNKS = D / 8;             // 16-byte pieces per bf16 row
  constexpr int AROW = D + 4;               // floats per row of the combine buffer
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(BF || ROPE == ROPE_NONE, "fused RoPE is built for bf16 only");

  float* s_acc = sm.acc;
  float (&s_m)[kDecWaves][16] = sm.m;
  float (&s_l)[kDecWaves][16] = sm.l;
  float (&s_lb)[kDecWaves][16] = sm.lb;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // the same value, known to be uniform
  const int n = lane & 15;  // MFMA N index: this lane's query row
  const int j = lane >> 4;  // lane group
  // key row (within a 16-key block) this lane feeds to the logits MFMA
  const int kkey = BF ? 4 * (n & 3) + (n >> 2) : n;

  const T* __restrict__ Qp = static_cast<const T*>(a.q);
  const T* __restrict__ Kp = static_cast<const T*>(a.k);
  const T* __restrict__ Vp = static_cast<const T*>(a.v);
  const int g = a.group;
  const bool block_in_page = DENSE || a.page_shift >= 4;  // an aligned 16-key block never crosses a page

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

    if constexpr (!DENSE) stage_pages(s_pages, a.page_indices, kbase, kv_lo, kv_hi, a.page_shift, tid, kDecThreads);
    __syncthreads();

    // ---- this lane's query row and its q fragment (MFMA B operand)
    const int rho = row_lo + n;
    const bool row_ok = rho < row_hi;
    const int qi = row_ok ? rho / g : 0;
    const int qu = row_ok ? rho % g : 0;
    const int qpos = L - qlen + qi;
    const T* qrow = Qp + int64_t(q0 + qi) * a.q_st + int64_t(h * g + qu) * a.q_sh;

    // RoPE positions: streaming = rank within the visible set (sinks, then the window)
    int lo_w = 0, n_s = 0;
    if constexpr (ROPE == ROPE_STREAMING) {
      lo_w = a.window > 0 ? max(0, qpos - a.window + 1) : 0;
      n_s = a.window > 0 ? min(a.sink, lo_w) : 0;
    }

    bf16x8 qh[BF ? NKS : 1];
    f16x8 qr[BF && ROPE != ROPE_NONE ? NKS : 1];   // rotated q in fp16 (fused RoPE)
    f16x8 qr2[BF && ROPE != ROPE_NONE ? NKS : 1];  // ... and what that rounding left out, in fp16
    float qf[BF ? 1 : NKS];
    if constexpr (BF) {
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        qh[s] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 8 * (4 * s + j)) : bf16x8{};
      }
      if constexpr (ROPE != ROPE_NONE) {
        int pq = ROPE == ROPE_STREAMING ? n_s + (qpos - lo_w) : qpos;
        pq = min(max(pq, 0), a.rope_n_pos - 1);
#pragma unroll
        for (int s = 0; s < HALF_KS; ++s) {
          float lo[8], hi[8];
          unpack_bf16x8(qh[s], lo);
          unpack_bf16x8(qh[s + HALF_KS], hi);
          rope8(lo, hi, reinterpret_cast<const float4*>(a.rope + (int64_t(pq) * (D / 2) + 8 * (4 * s + j)) * 2));
          qr[s] = to_f16x8(lo);
          qr[s + HALF_KS] = to_f16x8(hi);
          qr2[s] = f16_residual(lo, qr[s]);
          qr2[s + HALF_KS] = f16_residual(hi, qr[s + HALF_KS]);
        }
        if (!row_ok) {
#pragma unroll
          for (int s = 0; s < NKS; ++s) qr[s] = qr2[s] = f16x8{};
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < NKS; s += 4) {
        const float4 x = row_ok ? *reinterpret_cast<const float4*>(qrow + j * (D / 4) + s) : float4{0, 0, 0, 0};
        qf[s] = x.x;
        qf[s + 1] = x.y;
        qf[s + 2] = x.z;
        qf[s + 3] = x.w;
      }
    }

    const RowMask rm = row_mask(row_ok, qpos, kv_hi, a.causal, a.window, a.sink);
    // l_run: the fp32 sum of the probabilities (the LSE); lb_run: the same probabilities as the
    // bf16 PV operand holds them, which normalises O -- with bf16 P, dividing by l_run instead
    // would leave a dominant key's rounding (up to 2^-9 of its V row) in O
    float m_run = -INFINITY, l_run = 0.f, lb_run = 0.f;
    f32x4 acc[NACC];
#pragma unroll
    for (int e = 0; e < NACC; ++e) acc[e] = f32x4{0, 0, 0, 0};

    const int blk0 = kv_lo >> 4;
    const int nblk = ((kv_hi - 1) >> 4) - blk0 + 1;
    const int kmin = kv_lo, kmax = kv_hi - 1;

    // element offsets of key t of kv head h (K and V strides may differ)
    auto key_offsets = [&](int t, int64_t& ko, int64_t& vo) {
      ko = kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.k_sp, a.k_sh, a.k_st);
      if constexpr (SAME)
        vo = ko;
      else
        vo = kv_offset<DENSE>(s_pages, t, kbase, kv_lo, a.page_shift, h, a.v_sp, a.v_sh, a.v_st);
    };

    // masked, scaled logits -> probabilities; online-softmax state update
    auto softmax_update = [&](float* sv, float* p) {
      float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      bm = wave_max_xor16_32(bm);
      const bool grow = bm > m_run + kRescaleSlack || (m_run == -INFINITY && bm > -INFINITY);
      if (__any(grow)) {  // wave-uniform: rescale only when some row's max jumps
        const float m_new = grow ? bm : m_run;
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        lb_run *= alpha;
#pragma unroll
        for (int e = 0; e < NACC; ++e) acc[e] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
      l_run += (p[0] + p[1]) + (p[2] + p[3]);
    };

    if constexpr (BF) {
      // K: this lane's key row kkey, pieces 4s + j.  V: keys 4i + j (i = 0..3), piece n % CHUNKS.
      // Each V byte is read once, and one V load covers whole 128-byte lines (four full key rows),
      // so the V loads carry the non-temporal hint and their lines do not linger in L2.  A K load
      // covers half of each line it touches (four 16-byte pieces of a key row); the hint on K
      // measured slower (a streamed line may leave L2 before its other half is read).
      // A wave past its last block still issues a block's loads (`dummy`), so that every iteration
      // issues the same loads.  With a block inside one page they all read the block's first key
      // row (512 B of K and V instead of the block's 8 KB: on short items, where the block has
      // already left L2, re-reading it whole cost up to an eighth more traffic).
      auto load_block = [&](int b, bf16x8* kf, u32x4* vf, bool dummy) {
        const int tb = (blk0 + b) << 4;
        if (block_in_page) {
          const int t0 = min(max(tb, kmin), kmax);
          int64_t kb, vb;
          key_offsets(t0, kb, vb);  // one page id serves the whole block
          const int tk = dummy ? t0 : min(max(tb + kkey, kmin), kmax);
#pragma unroll
          for (int s = 0; s < NKS; ++s)
            kf[s] = *reinterpret_cast<const bf16x8*>(Kp + kb + int64_t(tk - t0) * a.k_st + 8 * (4 * s + j));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tv = dummy ? t0 : min(max(tb + 4 * i + j, kmin), kmax);
            vf[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(Vp + vb + int64_t(tv - t0) * a.v_st + 8 * (n % CHUNKS)));
          }
        } else {  // pages of < 16 keys: a dummy block is read whole (its rows may span pages)
          int64_t ko, vo;
          key_offsets(min(max(tb + kkey, kmin), kmax), ko, vo);
#pragma unroll
          for (int s = 0; s < NKS; ++s)
            kf[s] = *reinterpret_cast<const bf16x8*>(Kp + ko + 8 * (4 * s + j));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            key_offsets(min(max(tb + 4 * i + j, kmin), kmax), ko, vo);
            vf[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vp + vo + 8 * (n % CHUNKS)));
          }
        }
      };

      // (cos, sin) pairs of this lane's key row for the frequencies of its fragments 4s + j
      // (s < HALF_KS): four float4 per fragment
      constexpr int NCS = ROPE == ROPE_NONE ? 1 : 4 * HALF_KS;
      auto load_table = [&](int b, float4* cs) {
        if constexpr (ROPE != ROPE_NONE) {
          const int tk = min(max(((blk0 + b) << 4) + kkey, kmin), kmax);
          int pk = ROPE == ROPE_STREAMING ? (tk < n_s ? tk : n_s + (tk - lo_w)) : tk;
          pk = min(max(pk, 0), a.rope_n_pos - 1);
#pragma unroll
          for (int s = 0; s < HALF_KS; ++s) {
            const float4* c4 = reinterpret_cast<const float4*>(a.rope + (int64_t(pk) * (D / 2) + 8 * (4 * s + j)) * 2);
#pragma unroll
            for (int e = 0; e < 4; ++e) cs[4 * s + e] = c4[e];
          }
        }
      };

      // A wave's blocks are 4 x 16 keys apart, and inside an item the keys' positions are their
      // indices plus a constant (streaming ranks included: an item lies entirely in the window or
      // entirely in the sinks), so after the wave's first block the (cos, sin) pairs follow from
      // the previous block's by one rotation by 64 positions.  The first block reads the table, and
      // so does the second of wave 0 when the item starts inside a 16-key block: then wave 0's
      // first block holds keys before the item's range, whose positions are clamped.
      float4 step[NCS];
      if constexpr (ROPE != ROPE_NONE) {
        const int p64 = min(4 * 16, a.rope_n_pos - 1);
#pragma unroll
        for (int s = 0; s < HALF_KS; ++s) {
          const float4* c4 = reinterpret_cast<const float4*>(a.rope + (int64_t(p64) * (D / 2) + 8 * (4 * s + j)) * 2);
#pragma unroll
          for (int e = 0; e < 4; ++e) step[4 * s + e] = c4[e];
        }
      }
      auto next_table = [&](int b, float4* cs) {
        if constexpr (ROPE != ROPE_NONE) {
          const bool clamped_first = wave_u == 0 && (kv_lo & 15) != 0;
          if (b - wave_u < (clamped_first ? 2 : 1) * kDecWaves) {
            load_table(b, cs);
          } else {
#pragma unroll
            for (int q = 0; q < NCS; ++q) {
              const float4 c = cs[q], t = step[q];  // (cos, sin) of two frequencies
              cs[q] = float4{c.x * t.x - c.y * t.y, c.y * t.x + c.x * t.y, c.z * t.z - c.w * t.w, c.w * t.z + c.z * t.w};
            }
          }
        }
      };

      auto compute_block = [&](int b, bf16x8* kf, const u32x4* vf, const float4* cs) {
        const int tb = (blk0 + b) << 4;
        f32x4 st = {0, 0, 0, 0};
        if constexpr (ROPE == ROPE_NONE) {
#pragma unroll
          for (int s = 0; s < NKS; ++s) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qh[s], st, 0, 0, 0);
        } else {
#pragma unroll
          for (int s = 0; s < HALF_KS; ++s) {
            float lo[8], hi[8];
            unpack_bf16x8(kf[s], lo);
            unpack_bf16x8(kf[s + HALF_KS], hi);
            rope8(lo, hi, &cs[4 * s]);
            // first and second fp16 part of the rotated key, for its first (lo) and second (hi) half
            const f16x8 klo = to_f16x8(lo), khi = to_f16x8(hi);
            const f16x8 klo2 = f16_residual(lo, klo), khi2 = f16_residual(hi, khi);
            // the small terms first, then the main product
            st = __builtin_amdgcn_mfma_f32_16x16x32_f16(klo2, qr[s], st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_16x16x32_f16(klo, qr2[s], st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_16x16x32_f16(klo, qr[s], st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_16x16x32_f16(khi2, qr[s + HALF_KS], st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_16x16x32_f16(khi, qr2[s + HALF_KS], st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_16x16x32_f16(khi, qr[s + HALF_KS], st, 0, 0, 0);
          }
        }
        // st[i]: logit of key tb + 4i + j for query row n
        float sv[4], p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tb + 4 * i + j;
          sv[i] = (row_sees(rm, t) & (t >= kv_lo)) ? st[i] * a.scale_log2 : -INFINITY;
        }
        softmax_update(sv, p);
        u32x2 pw;
        pw[0] = pack_bf16x2(p[0], p[1]);
        pw[1] = pack_bf16x2(p[2], p[3]);
        lb_run = add_bf16x2(pw[1], add_bf16x2(pw[0], lb_run));
        const i16x4 pb = __builtin_bit_cast(i16x4, pw);
        // A operand e: element e of this lane's four V pieces = V[key 4i+j][d = 8*(n%CHUNKS) + e]
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(gather_e(vf[0], vf[1], vf[2], vf[3], e), pb, acc[e],
                                                              0, 0, 0);
      };

      // Two register sets: the next block's loads are in flight while the current one is consumed.
      // Every iteration issues the same loads in the same order -- a wave without a next block
      // issues dummy loads from its current block -- so the wait before a block's math only has
      // to let the next block's loads (and, with RoPE, nothing else) stay outstanding; a load
      // skipped on some path would force a wait for everything issued so far.  The RoPE table
      // values of a block are requested before the next block's K/V for the same reason.
      bf16x8 ka[NKS], kb2[NKS];
      u32x4 va[4], vb2[4];
      float4 cs[NCS];
      int b = wave_u;
      if (b < nblk) load_block(b, ka, va, false);
      for (; b < nblk; b += 2 * kDecWaves) {
        const int b1 = b + kDecWaves;
        next_table(b, cs);
        load_block(b1 < nblk ? b1 : b, kb2, vb2, b1 >= nblk);
        compute_block(b, ka, va, cs);
        if (b1 >= nblk) break;
        const int b2 = b1 + kDecWaves;
        next_table(b1, cs);
        load_block(b2 < nblk ? b2 : b1, ka, va, b2 >= nblk);
        compute_block(b1, kb2, vb2, cs);
      }
    } else {
      for (int b = wave; b < nblk; b += kDecWaves) {
        const int tb = (blk0 + b) << 4;
        int64_t ko, vo;
        key_offsets(min(max(tb + n, kmin), kmax), ko, vo);
        float kf[NKS];
#pragma unroll
        for (int s = 0; s < NKS; s += 4) {
          const float4 x = *reinterpret_cast<const float4*>(Kp + ko + j * (D / 4) + s);
          kf[s] = x.x;
          kf[s + 1] = x.y;
          kf[s + 2] = x.z;
          kf[s + 3] = x.w;
        }
        f32x4 st = {0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < NKS; ++s) st = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[s], qf[s], st, 0, 0, 0);
        // st[i]: logit of key tb + 4j + i
        float sv[4], p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tb + 4 * j + i;
          sv[i] = (row_sees(rm, t) & (t >= kv_lo)) ? st[i] * a.scale_log2 : -INFINITY;
        }
        softmax_update(sv, p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          key_offsets(min(max(tb + 4 * j + i, kmin), kmax), ko, vo);
#pragma unroll
          for (int db = 0; db < NACC; ++db)
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(static_cast<float>(Vp[vo + 16 * db + n]), p[i], acc[db],
                                                           0, 0, 0);
        }
      }
    }

    // ---- combine the four waves' states through LDS (each lane owns query row n)
    l_run = wave_sum_xor16_32(l_run);
    lb_run = BF ? wave_sum_xor16_32(lb_run) : l_run;  // fp32 P (f32 inputs) needs no second sum
    if (j == 0) {
      s_m[wave][n] = m_run;
      s_l[wave][n] = l_run;
      s_lb[wave][n] = lb_run;
    }
    __syncthreads();
    {
      const float M = fmaxf(fmaxf(s_m[0][n], s_m[1][n]), fmaxf(s_m[2][n], s_m[3][n]));
      const float my = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
      float* crow = s_acc + (wave * 16 + n) * AROW;
      if constexpr (BF) {
        // acc[e][i] holds column 8 * (4j + i) + e; with D = 64 lane groups j >= 2 repeat j - 2
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 4 * j + i;
          if (c < CHUNKS) {
            *reinterpret_cast<float4*>(crow + 8 * c) =
                float4{acc[0][i] * my, acc[1][i] * my, acc[2][i] * my, acc[3][i] * my};
            *reinterpret_cast<float4*>(crow + 8 * c + 4) =
                float4{acc[4][i] * my, acc[5][i] * my, acc[6][i] * my, acc[7][i] * my};
          }
        }
      } else {
        // acc[db][i] holds column 16 db + 4j + i
#pragma unroll
        for (int db = 0; db < NACC; ++db)
          *reinterpret_cast<float4*>(crow + 16 * db + 4 * j) =
              float4{acc[db][0] * my, acc[db][1] * my, acc[db][2] * my, acc[db][3] * my};
      }
    }
    __syncthreads();
    const int nrows = row_hi - row_lo;
    for (int e = tid; e < nrows * (D / 4); e += kDecThreads) {
      const int rr = e / (D / 4);
      const int c4 = (e % (D / 4)) * 4;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, s_m[w][rr]);
      float Lsum = 0.f, Lb = 0.f;
      float4 o = {0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        if (s_m[w][rr] != -INFINITY) {
          const float sc = __builtin_amdgcn_exp2f(s_m[w][rr] - M);
          Lsum += s_l[w][rr] * sc;
          Lb += s_lb[w][rr] * sc;
        }
        const float4 x = *reinterpret_cast<const float4*>(s_acc + (w * 16 + rr) * AROW + c4);
        o.x += x.x;
        o.y += x.y;
        o.z += x.z;
        o.w += x.w;
      }
      const float inv = Lb > 0.f ? 1.f / Lb : 0.f;
      o.x *= inv;
      o.y *= inv;
      o.z *= inv;
      o.w *= inv;
      const float lse = Lsum > 0.f ? (M + __log2f(Lsum)) * 0.69314718055994531f : -INFINITY;
      const int row = row_lo + rr;
      if (slot < 0) {
        const int tok = q0 + row / g;
        const int qhd = h * g + row % g;
        const int64_t oo = int64_t(tok) * a.o_st + int64_t(qhd) * a.o_sh + c4;
        if (a.out_bf16) {
          uint2 pk2 = {pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
          *reinterpret_cast<uint2*>(static_cast<__bf16*>(a.out) + oo) = pk2;
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + oo) = o;
        }
        if (c4 == 0) a.lse[int64_t(tok) * a.lse_st + qhd] = lse;
      } else {
        store_part4(a.part_o + (int64_t(slot) * part_rows + rr) * D + c4, o.x, o.y, o.z, o.w, a.fused_merge);
        if (c4 == 0) store_part(a.part_lse + int64_t(slot) * part_rows + rr, lse, a.fused_merge);
      }
    }
    if (slot >= 0 && a.fused_merge) finish_split_chunk<D>(a, slot, tid, kDecThreads, s_last);
    __syncthreads();
  }
}

}  // namespace bsk
