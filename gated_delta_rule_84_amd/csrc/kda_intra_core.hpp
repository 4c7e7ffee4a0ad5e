// Intra-chunk steps of a 64-token chunk: everything that does not depend on
// the recurrent state.  Four waves cooperate on a chunk; wave i owns the
// chunk's 16-token sub-tile i and keeps that sub-tile's rows of q, k and of
// the log-decay prefix in registers.  The steps are shared by the standalone
// intra-chunk kernel (record to HBM) and the fused kernel (record straight
// into the scan's LDS image); the caller supplies the synchronisation between
// steps and the destination of each record part.
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3).  Section 2.1 gives the chunked output
// O = (Gamma . Q) S + Tril[(Q . Gamma)(K / Gamma)^T](U - W S); U and W are the
// UT-transform pair (I + StrictTril(Diag(beta)(K . Gamma)(K / Gamma)^T))^{-1}
// applied to Diag(beta) V and Diag(beta)(K . Gamma).  Section 2.2: the chunk is
// cut into 16-token sub-tiles and, because the K3 decay keeps a sub-tile's
// cumulative log-decay within (-80, 0), every causal sub-tile block --
// diagonal blocks included -- is a dense matrix product of decay-scaled
// factors.  Sub-tile i is anchored at its 8th token, B_i = G[16 i + 7], so
// the factors of every block stay within e^{+-40}:
//     A(i, i) = (K_i . e^{G_i - B_i}) (K_i . e^{B_i - G_i})^T
//     A(i, j) = (K_i . e^{G_i - B_i} . e^{B_i - B_j}) (K_j . e^{B_j - G_j})^T,  j < i.
// Precision (bf16 path): A_qk's diagonal blocks are fp32 products of the fp32
// factors (fp32 MFMA); every other block is a plain bf16 product.  The fp32
// path uses fp32 MFMA throughout.  The log-decay is carried in base-2 units
// (G log2(e)), so every decay factor is one exp2.
//
// The products are formed transposed -- column factors as the A operand, row
// factors as the B operand -- so that each lane ends up with four consecutive
// columns of one *row* of A_kk, A_qk and T.  Those rows go to the record with
// 8-byte stores and serve directly as A operands of the fp32 MFMAs of the UT
// inverse.  Kd^T is transposed the other way by multiplying with a 0/1
// selection matrix on MFMA (exact).
//
// Record parts (layout in kda_params.hpp, precision and scaling in RecOps):
//   qg = q^ . Gamma, kg = -(k^ . Gamma), kdt = (k^ . Gamma_last / Gamma)^T,
//   tb = T Diag(beta) with T = (I + Diag(beta) StrictTril(A_kk))^{-1},
//   aq = Tril(A_qk) (diagonal included), gam = Gamma_last.
#pragma once

#include "kda_chunk_prologue.hpp"

namespace kda {

// 8 fp32 values as the fp32 operand of one 32-wide K-step (eight 16x16x4 MFMAs).
__device__ __forceinline__ f32x8 f32x8_of(const float* x) {
  return f32x8{x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
}

template <typename T>
struct APolicy;
template <>
struct APolicy<uint16_t> {  // bf16 path
  using Plain = bf16x8;
  static __device__ __forceinline__ Plain plain(const float* x) { return pack8_bf16(x); }
  static __device__ __forceinline__ f32x4 mma(const Plain& a, const Plain& b, f32x4 acc) { return mma32(a, b, acc); }
  static __device__ __forceinline__ Plain ld(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
};
template <>
struct APolicy<float> {  // fp32 path
  using Plain = f32x8;
  static __device__ __forceinline__ f32x8 plain(const float* x) { return f32x8_of(x); }
  static __device__ __forceinline__ f32x4 mma(const f32x8& a, const f32x8& b, f32x4 acc) { return mma32(a, b, acc); }
  static __device__ __forceinline__ f32x8 ld(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
};

__device__ __forceinline__ int slot_row64(int p) { return (p & 32) + slot_row(p & 31); }

// index of the pair (i, j), i > j, in 0..5
__device__ __forceinline__ int pair_index(int i, int j) { return (i * (i - 1)) / 2 + j; }

// 0/1 selection operand (B side): column n of the product picks channel
// 32 kk + 16 half + n of the A operand's K-step, so that C = A . Sel puts
// A's rows on C's rows and its channels on the lanes.
template <typename P>
__device__ __forceinline__ P select_operand(int n, int g, int half) {
  P s;
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = (g == (n >> 2) && j == 4 * half + (n & 3)) ? 1.0f : 0.0f;
  return s;
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS work areas of the intra-chunk steps (all per chunk):
//   loc7 [4][D]  prefix at each sub-tile's anchor row   tot [4][D] sub-tile totals
//   Et   [6][D]  e^{B_i - B_j}, pairs i > j             eB  [4][D] e^{B_i}
//   eL   [4][D]  e^{G_last - B_i}                       betas [64]
//   KC   [48][KP] column factors of sub-tiles 0..2 (element type T)
//   Tm   [64][68] the UT inverse T, fp32, row-major
// tot is dead once the tables are built; loc7 is read until the factors are
// formed (while KC is written).
template <typename T>
struct IntraScratch {
  float* loc7;
  float* tot;
  float* Et;
  float* eB;
  float* eL;
  float* betas;
  T* KC;
  float* Tm;
};

// The steps, in order (the caller synchronises the four waves where marked):
//   load -> prefix | tables | factors | offdiag, solve | level 1 | 2 | 3 | tb_pass
// PQE / PKE: row pitches (elements) of the record's [64][D] parts (qg, kg) and
// of its 64-column parts (kdt, tb, aq), when the record is an LDS image
// (UNITS = false); with UNITS the record is the workspace's unit layout
// (rec_units: each wave store writes 1 KB of consecutive bytes), written
// through `sink` with device-scope stores (see RecSink).
//
// SP: Kimi Linear's unbounded decay g = -e^{A_h} Softplus(z), the map the K3
// blog's section 2.2 replaces.  Without the sub-tile bound the factors of a
// diagonal block overflow, so (as section 2.2 describes for Kimi Linear) the
// diagonal blocks are computed pair by pair, with e^{G_r - G_c} <= 1 per
// channel; the off-diagonal blocks are anchored at sub-tile ends so that
// every factor is at most 1:
//     A(i, j) = (K_i . e^{G_i - E_{i-1}} . e^{E_{i-1} - E_j}) (K_j . e^{E_j - G_j})^T,
// E_j the log-decay at the end of sub-tile j (E_{i-1} - E_j = the totals of
// sub-tiles j + 1 .. i - 1).
template <typename T, int D, int PQE, int PKE, bool SP = false, bool UNITS = false>
struct IntraCore {
  using AP = APolicy<T>;
  using R8 = Run8<T>;
  using RO = RecOps<T>;                          // record precision
  using RE = typename RO::Elem;                  // record element (fp16 bits or fp32)
  using Rec4 = decltype(RO::pack4(f32x4{}));     // 4 record elements in registers
  static constexpr int KS = D / 32;
  static constexpr int KP = D + 16 / (int)sizeof(T);  // KC row pitch (elements)
  static constexpr int LP = 68;                       // Tm row pitch (floats)

  int ti, n, g4, r;
  bool rvalid;
  typename R8::Raw qraw[KS], kraw[KS], zraw[KS];
  float beta_r, rq, rk;
  float P[KS][8];
  float KR[KS][8], QR[KS][8];  // row factors (kept for the off-diagonal blocks)
  f32x4 akk_d, aqk_d, akk[3], aqk[3], tii;
  Rec4 kd[KS][2];              // Kd^T pieces awaiting their store
  Rec4 aqs[4];                 // Tril(A_qk) row pieces (4 columns of each block) awaiting their store
  RecSink sink;                // UNITS: the record's device-scope stores

  // 8 fp32 values as 8 record elements through the sink (one or two units)
  static __device__ __forceinline__ void sink_store8(const RecSink& k, RE* p, const float* x) {
    if constexpr (sizeof(RE) == 2) {
      k.st16(p, RO::pack8(x));
    } else {
      k.st16(p, u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])});
      k.st16(p + 4, u32x4{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])});
    }
  }

  // 8 fp32 values as 8 record elements at p (an LDS image)
  static __device__ __forceinline__ void rec_store8(RE* p, const float* x) {
    if constexpr (sizeof(RE) == 2) {
      *reinterpret_cast<u32x4*>(p) = RO::pack8(x);
    } else {
      *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
  }

  __device__ __forceinline__ void init(int wave, int lane) {
    ti = wave;
    n = lane & 15;
    g4 = lane >> 4;
    r = 16 * ti + n;
  }

  // This wave's sub-tile rows of q, k, z (operand layout) and beta.  Rows past
  // the end of the sequence re-read the last row and are masked later.
  __device__ __forceinline__ void load(const IntraParams& p, int b, int h, int tok0, int nvalid) {
    const int64_t tok_stride = token_stride(p.head_first, p.H, D);
    const int64_t row0 = token_base(p.head_first, b, h, p.T, p.H, D) + tok0 * tok_stride;
    rvalid = r < nvalid;
    const int64_t rowp = row0 + min(r, nvalid - 1) * tok_stride;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      qraw[kk] = R8::load(static_cast<const T*>(p.q) + rowp, kk, g4);
      kraw[kk] = R8::load(static_cast<const T*>(p.k) + rowp, kk, g4);
      zraw[kk] = R8::load(static_cast<const T*>(p.z) + rowp, kk, g4);
    }
    const int64_t bi = token_base(p.head_first, b, h, p.T, p.H, 1) + (tok0 + r) * token_stride(p.head_first, p.H, 1);
    beta_r = rvalid ? Elem<T>::to_f32(static_cast<const T*>(p.beta)[bi]) : 0.0f;
  }

  // Decay prefix within the sub-tile (base 2); anchor rows and totals to LDS;
  // beta to LDS; inverse norms.
  __device__ __forceinline__ void prefix(const IntraParams& p, int h, const IntraScratch<T>& s) {
    if (g4 == 0) s.betas[r] = beta_r;
    subtile_decay_prefix<T, KS, SP>(zraw, p.A[h], p.g_min, kLog2e, rvalid, P);
    if (n == 7)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) put_run8(s.loc7 + ti * D, kk, g4, P[kk]);
    if (n == 15)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) put_run8(s.tot + ti * D, kk, g4, P[kk]);
    const float nq = row_inv_norm<T, KS>(qraw, p.l2norm, p.l2_eps);
    const float nk = row_inv_norm<T, KS>(kraw, p.l2norm, p.l2_eps);
    rq = rvalid ? nq * p.q_scale : 0.0f;
    rk = rvalid ? nk : 0.0f;
  }

  // Per-channel tables from the sub-tile totals and anchors (thread t of
  // nthreads, all four waves), base 2:  G of sub-tile i = off_i + prefix,
  // off_i = sum_{j < i} tot_j;  B_i = off_i + loc7_i.  Gamma_last goes to gam.
  template <int NTHREADS>
  static __device__ __forceinline__ void tables(int t, const IntraScratch<T>& s, float* gam,
                                                const RecSink* sink = nullptr) {
    constexpr int TPC = NTHREADS / D;
    const int ch = t % D, part = t / D;
    float off[4], Bv[4], Ev[4];
    off[0] = 0.0f;
#pragma unroll
    for (int i = 1; i < 4; ++i) off[i] = off[i - 1] + s.tot[(i - 1) * D + ch];
    const float glast = off[3] + s.tot[3 * D + ch];
    // K3: one anchor per sub-tile (its 8th row) for rows and columns.  SP:
    // rows anchored at the previous sub-tile's end (off_i), columns at their
    // own sub-tile's end (off_{i + 1}).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Bv[i] = SP ? off[i] : off[i] + s.loc7[i * D + ch];
      Ev[i] = SP ? (i < 3 ? off[i + 1] : glast) : Bv[i];
    }
    // 15 items per channel, item % TPC == part for this thread; every index
    // is a compile-time constant and `part` is uniform over a wave (D >= 64)
#pragma unroll
    for (int item = 0; item < 15; ++item) {
      if (item % TPC != part) continue;
      if (item < 4) {
        s.eB[item * D + ch] = hw_exp2(Bv[item] + RO::kLog2Up);  // the record's factor on q^ . Gamma, k^ . Gamma
      } else if (item < 8) {
        s.eL[(item - 4) * D + ch] = hw_exp2(glast - Ev[item - 4] - RO::kLog2Up);  // and its inverse on Kd
      } else if (item < 14) {
        const int pi = item - 8;  // pair index -> (i, j)
        const int i = (pi < 1) ? 1 : (pi < 3) ? 2 : 3;
        const int j = pi - pair_index(i, 0);
        s.Et[pi * D + ch] = hw_exp2(Bv[i] - Ev[j]);
      } else {
        if constexpr (UNITS)
          sink->st4(gam + ch, hw_exp2(glast));
        else
          gam[ch] = hw_exp2(glast);
      }
    }
  }

  // Own sub-tile: factors, qg / kg rows, column factors, Kd^T (held), the
  // diagonal blocks and L_ii = Diag(beta) StrictTril(A_kk(i, i)) staged in Tm.
  __device__ __forceinline__ void factors(const IntraScratch<T>& s, T* qg, T* kg) {
    akk_d = zero4();
    aqk_d = zero4();
    const typename RO::V8 sel0 = select_operand<typename RO::V8>(n, g4, 0);
    const typename RO::V8 sel1 = select_operand<typename RO::V8>(n, g4, 1);
    float KN[SP ? KS : 1][8], QN[SP ? KS : 1][8];  // SP: normalised rows for the pairwise diagonal
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      float p7[8], eb[8], el[8];
      // K3: the anchor row; SP: the sub-tile total (the column anchor)
      lds_run8((SP ? s.tot : s.loc7) + ti * D, kk, g4, p7);
      lds_run8(s.eB + ti * D, kk, g4, eb);
      lds_run8(s.eL + ti * D, kk, g4, el);
      float kc[8], xq[8], xk[8], xd[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // K3: rf = e^{G_r - B_i}, cf = e^{B_i - G_r}.  SP: rf = e^{G_r - E_{i-1}}
        // = 2^{P}, cf = e^{E_i - G_r} = 2^{tot - P}, both at most 1.
        const float d = P[kk][j] - p7[j];  // log2 units
        const float rf = hw_exp2(SP ? P[kk][j] : d);
        const float cf = hw_exp2(-d);
        const float kn = R8::get(kraw[kk], j) * rk;  // normalised k, q
        const float qn = R8::get(qraw[kk], j) * rq;
        if constexpr (SP) {
          KN[kk][j] = kn;
          QN[kk][j] = qn;
        }
        KR[kk][j] = kn * rf;
        QR[kk][j] = qn * rf;
        kc[j] = kn * cf;
        xq[j] = QR[kk][j] * eb[j];   // q^ . Gamma
        xk[j] = -KR[kk][j] * eb[j];  // -(k^ . Gamma)
        xd[j] = kc[j] * el[j];       // k^ . Gamma_last / Gamma
      }
      if constexpr (UNITS) {
        const int pc = (ti * KS + kk) * 64 + 16 * g4 + n;  // piece of this lane
        sink_store8(sink, qg + 8 * pc, xq);
        sink_store8(sink, kg + 8 * pc, xk);
      } else {
        rec_store8(qg + r * PQE + 32 * kk + 8 * g4, xq);
        rec_store8(kg + r * PQE + 32 * kk + 8 * g4, xk);
      }
      if (ti < 3) store8<T>(s.KC + r * KP + 32 * kk + 8 * g4, kc);  // column factors for later sub-tiles
      {
        // lane (n, g4) receives Kd[16 ti + 4 g4 + i][32 kk + 16 half + n]
        // (a 0/1 product in the record's precision: exact)
        const typename RO::V8 xdp = RO::plain(xd);
        kd[kk][0] = RO::pack4(RO::mma(xdp, sel0, zero4()));
        kd[kk][1] = RO::pack4(RO::mma(xdp, sel1, zero4()));
      }
      if constexpr (!SP) {
        // transposed diagonal blocks: lane (n, g4) gets row n, columns 4 g4 + i
        akk_d = AP::mma(AP::plain(kc), AP::plain(KR[kk]), akk_d);
        aqk_d = mma32(f32x8_of(kc), f32x8_of(QR[kk]), aqk_d);
      }
    }
    if constexpr (SP) pairwise_diagonal(s, KN, QN);
    f32x4 lv;
#pragma unroll
    for (int i = 0; i < 4; ++i) lv[i] = (4 * g4 + i < n) ? beta_r * akk_d[i] : 0.0f;
    *reinterpret_cast<f32x4*>(s.Tm + r * LP + 16 * ti + 4 * g4) = lv;
  }

  // SP diagonal block, pair by pair: for c <= n,
  //     A_kk(i, i)[n][c] = sum_ch kn_n kn_c e^{G_n - G_c},  A_qk likewise with qn_n,
  // every exponent <= 0 (a sub-tile's prefix P is non-increasing).  Each lane
  // sums its 32 channels; row c's prefix and keys come through a strip of LDS
  // inside this sub-tile's own rows of Tm (wave-private until the workgroup
  // synchronises after the factors), one K-step at a time; the four lane
  // groups of a row then add their partial sums.
  template <int KN_ROWS>
  __device__ __forceinline__ void pairwise_diagonal(const IntraScratch<T>& s, const float (&kn)[KN_ROWS][8],
                                                    const float (&qn)[KN_ROWS][8]) {
    static_assert(16 * 64 <= 16 * LP, "strip inside the sub-tile's rows of Tm");
    float* strip = s.Tm + (16 * ti) * LP;  // [16 rows][32 P | 32 k] of one K-step
    float ak[16], aq[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) ak[c] = aq[c] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      __builtin_amdgcn_wave_barrier();  // every lane has read the previous K-step's strip
      *reinterpret_cast<float4*>(strip + n * 64 + 8 * g4) = make_float4(P[kk][0], P[kk][1], P[kk][2], P[kk][3]);
      *reinterpret_cast<float4*>(strip + n * 64 + 8 * g4 + 4) = make_float4(P[kk][4], P[kk][5], P[kk][6], P[kk][7]);
      *reinterpret_cast<float4*>(strip + n * 64 + 32 + 8 * g4) = make_float4(kn[kk][0], kn[kk][1], kn[kk][2], kn[kk][3]);
      *reinterpret_cast<float4*>(strip + n * 64 + 32 + 8 * g4 + 4) =
          make_float4(kn[kk][4], kn[kk][5], kn[kk][6], kn[kk][7]);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float4 p0 = *reinterpret_cast<const float4*>(strip + c * 64 + 8 * g4);
        const float4 p1 = *reinterpret_cast<const float4*>(strip + c * 64 + 8 * g4 + 4);
        const float4 k0 = *reinterpret_cast<const float4*>(strip + c * 64 + 32 + 8 * g4);
        const float4 k1 = *reinterpret_cast<const float4*>(strip + c * 64 + 32 + 8 * g4 + 4);
        const float pc[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        const float kc[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // c > n gives positive exponents: clamped (those entries are masked later)
          const float w = kc[j] * hw_exp2(fminf(P[kk][j] - pc[j], 0.0f));
          ak[c] = __builtin_fmaf(kn[kk][j], w, ak[c]);
          aq[c] = __builtin_fmaf(qn[kk][j], w, aq[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      ak[c] += __shfl_xor(ak[c], 16);
      ak[c] += __shfl_xor(ak[c], 32);
      aq[c] += __shfl_xor(aq[c], 16);
      aq[c] += __shfl_xor(aq[c], 32);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      akk_d[i] = (g4 == 0) ? ak[i] : (g4 == 1) ? ak[4 + i] : (g4 == 2) ? ak[8 + i] : ak[12 + i];
      aqk_d[i] = (g4 == 0) ? aq[i] : (g4 == 1) ? aq[4 + i] : (g4 == 2) ? aq[8 + i] : aq[12 + i];
    }
    __builtin_amdgcn_wave_barrier();  // the strip is read out before L_ii overwrites these rows
  }

  // Kd^T pieces to the record: record position of the four tokens
  // 16 ti + 4 g4 + 0..3 inside a 64-token row.
  __device__ __forceinline__ void store_kd(T* kdt) const {
    const int tpos = 32 * (ti >> 1) + 8 * g4 + 4 * (ti & 1);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (UNITS) {
        T* dst = kdt + 8 * ((ti * KS + kk) * 64 + 16 * g4 + n);  // the two pieces side by side
        if constexpr (sizeof(T) == 2) {
          sink.st16(dst, u32x4{kd[kk][0].x, kd[kk][0].y, kd[kk][1].x, kd[kk][1].y});
        } else {
          sink.st16(dst, __builtin_bit_cast(u32x4, kd[kk][0]));
          sink.st16(dst + 4, __builtin_bit_cast(u32x4, kd[kk][1]));
        }
      } else {
        *reinterpret_cast<Rec4*>(kdt + (32 * kk + n) * PKE + tpos) = kd[kk][0];
        *reinterpret_cast<Rec4*>(kdt + (32 * kk + 16 + n) * PKE + tpos) = kd[kk][1];
      }
    }
  }

  // Off-diagonal blocks (ti, jt), jt < ti: plain products; then this wave's
  // rows of Tril(A_qk) packed for the record.
  __device__ __forceinline__ void offdiag(const IntraScratch<T>& s) {
#pragma unroll
    for (int jt = 0; jt < 3; ++jt) {
      akk[jt] = aqk[jt] = zero4();
      if (jt < ti) {
        const int pi = pair_index(ti, jt);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          float e8[8], xk[8], xq[8];
          lds_run8(s.Et + pi * D, kk, g4, e8);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            xk[j] = KR[kk][j] * e8[j];
            xq[j] = QR[kk][j] * e8[j];
          }
          const typename AP::Plain aop = AP::ld(s.KC + (16 * jt + n) * KP + 32 * kk + 8 * g4);
          akk[jt] = AP::mma(aop, AP::plain(xk), akk[jt]);
          aqk[jt] = AP::mma(aop, AP::plain(xq), aqk[jt]);
        }
      }
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x4 a;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = (jt == ti) ? ((4 * g4 + i <= n) ? aqk_d[i] : 0.0f) : (jt < ti ? aqk[jt < 3 ? jt : 0][i] : 0.0f);
      aqs[jt] = RO::pack4(a);
    }
  }

  // Tril(A_qk) rows to the record: the column pairs p <= ti / 2 of this row
  // tile, blocks 2 p and 2 p + 1 side by side (the upper blocks (0, 1) and
  // (2, 3), which the scan multiplies as part of its K-steps, are zeros).
  __device__ __forceinline__ void store_aq(RE* aq) const {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (p <= (ti >> 1)) {
        if constexpr (UNITS) {
          RE* dst = aq + 8 * (64 * aq_group(ti, p) + 16 * g4 + n);
          if constexpr (sizeof(RE) == 2) {
            sink.st16(dst, u32x4{aqs[2 * p].x, aqs[2 * p].y, aqs[2 * p + 1].x, aqs[2 * p + 1].y});
          } else {
            sink.st16(dst, __builtin_bit_cast(u32x4, aqs[2 * p]));
            sink.st16(dst + 4, __builtin_bit_cast(u32x4, aqs[2 * p + 1]));
          }
        } else {
          RE* dst = aq + r * PKE + 32 * p + 8 * g4;
          *reinterpret_cast<Rec4*>(dst) = aqs[2 * p];
          *reinterpret_cast<Rec4*>(dst + 4) = aqs[2 * p + 1];
        }
      }
    }
  }

  // T_ii = (I + L_ii)^{-1}, row n, by back substitution over the columns:
  // T (I + L) = I gives T[n][c] = delta_nc - sum_{s > c} T[n][s] L[s][c]: once
  // T[n][s] is final its multiple of row s of L is removed from every column
  // c < s.  All four lane groups solve row n; group g4 keeps columns 4 g4 + i.
  // Then the L rows of the off-diagonal blocks (A operands of the levels).
  __device__ __forceinline__ void solve(const IntraScratch<T>& s) {
    const float* Ls = s.Tm + (16 * ti) * LP + 16 * ti;
    float x[16];
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) x[cc] = (cc == n) ? 1.0f : 0.0f;
#pragma unroll
    for (int st = 15; st >= 1; --st) {
      float lrow[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        if (4 * q4 < st) {
          const float4 v = *reinterpret_cast<const float4*>(Ls + st * LP + 4 * q4);
          lrow[4 * q4] = v.x;
          lrow[4 * q4 + 1] = v.y;
          lrow[4 * q4 + 2] = v.z;
          lrow[4 * q4 + 3] = v.w;
        }
      }
      const float xs = x[st];
#pragma unroll
      for (int cc = 0; cc < st; ++cc) x[cc] -= xs * lrow[cc];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      tii[i] = (g4 == 0) ? x[i] : (g4 == 1) ? x[4 + i] : (g4 == 2) ? x[8 + i] : x[12 + i];
    __builtin_amdgcn_wave_barrier();  // every lane of the wave has read L_ii
    *reinterpret_cast<f32x4*>(s.Tm + r * LP + 16 * ti + 4 * g4) = tii;
#pragma unroll
    for (int jt = 0; jt < 3; ++jt)
#pragma unroll
      for (int i = 0; i < 4; ++i) akk[jt][i] *= beta_r;
  }

  // Off-diagonal blocks of T at distance dist: T_ij = -T_ii sum_{m=j}^{i-1} L_im T_mj,
  // fp32 MFMA 16x16x4 with K index 4 g + t in step t: the A operands are the
  // rows this lane holds (L_im, T_ii), the B operands columns (T_mj from LDS,
  // and the accumulator P as produced).  Every T_mj with m - j < dist must be
  // in LDS.
  __device__ __forceinline__ void level(int dist, const IntraScratch<T>& s) const {
    if (ti >= dist) {
      const int j = ti - dist;
      f32x4 Pm = zero4();
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        if (m >= j && m < ti) {
#pragma unroll
          for (int t = 0; t < 4; ++t) Pm = mfma4(akk[m][t], s.Tm[(16 * m + 4 * g4 + t) * LP + 16 * j + n], Pm);
        }
      }
      f32x4 Tn = zero4();
#pragma unroll
      for (int t = 0; t < 4; ++t) Tn = mfma4(tii[t], Pm[t], Tn);
      // lane holds column 16 j + n, rows 16 ti + 4 g4 + i
#pragma unroll
      for (int i = 0; i < 4; ++i) s.Tm[(16 * ti + 4 * g4 + i) * LP + 16 * j + n] = -Tn[i];
    }
  }

  // tb = T Diag(beta), columns in slot order; upper blocks are zero (thread t
  // of NTHREADS, all four waves; every block of T in LDS).
  template <int NTHREADS>
  static __device__ __forceinline__ void tb_pass(int t, const IntraScratch<T>& s, T* tb,
                                                 const RecSink* sink = nullptr) {
    for (int idx = t; idx < kChunk * 8; idx += NTHREADS) {
      const int rr = idx >> 3, pg = idx & 7;
      if (UNITS && rr < 32 && pg >= 4) continue;  // never read: not stored
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sc = slot_row64(8 * pg + j);
        x[j] = ((sc >> 4) <= (rr >> 4)) ? s.Tm[rr * LP + sc] * s.betas[sc] : 0.0f;
      }
      if constexpr (UNITS)
        sink_store8(*sink, tb + (rr < 32 ? 32 * rr : 1024 + 64 * (rr - 32)) + 8 * pg, x);
      else
        rec_store8(tb + rr * PKE + 8 * pg, x);
    }
  }
};

}  // namespace kda
