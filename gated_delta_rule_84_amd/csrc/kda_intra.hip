// Intra-chunk kernel: everything of a 64-token chunk that does not depend on
// the recurrent state.  One workgroup (4 waves) per (chunk, head, batch);
// wave i owns the chunk's 16-token sub-tile i and keeps that sub-tile's rows
// of q, k and of the log-decay prefix in registers.
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
// Precision (bf16 path): A_qk's diagonal blocks multiply hi/lo bf16 splits of
// both factors (three MFMAs per step); every other block is a plain bf16
// product.  The fp32 path uses fp32 MFMA throughout.
//
// The products are formed transposed -- column factors as the A operand, row
// factors as the B operand -- so that each lane ends up with four consecutive
// columns of one *row* of A_kk, A_qk and T.  Those rows go to the record with
// 8-byte stores and serve directly as A operands of the fp32 MFMAs of the UT
// inverse.  Kd^T is transposed the other way by multiplying with a 0/1
// selection matrix on MFMA (exact).
//
// Outputs (one record per chunk, layout in kda_params.hpp):
//   qg = q^ . Gamma, kg = -(k^ . Gamma), kdt = (k^ . Gamma_last / Gamma)^T,
//   tb = T Diag(beta) with T = (I + Diag(beta) StrictTril(A_kk))^{-1},
//   aq = Tril(A_qk) (diagonal included), gam = Gamma_last.
#include "kda_chunk_prologue.hpp"

namespace kda {

template <typename T>
struct APolicy;
template <>
struct APolicy<uint16_t> {  // bf16 path
  struct Split {
    bf16x8 hi, lo;
  };
  using Plain = bf16x8;
  static __device__ __forceinline__ Split split(const float* x) {
    Split o;
    split8_bf16(x, o.hi, o.lo);
    return o;
  }
  static __device__ __forceinline__ Plain plain(const float* x) { return pack8_bf16(x); }
  static __device__ __forceinline__ f32x4 mma(const Split& a, const Split& b, f32x4 acc) {
    return mma32_x3(a.hi, a.lo, b.hi, b.lo, acc);
  }
  static __device__ __forceinline__ f32x4 mma(const Plain& a, const Plain& b, f32x4 acc) { return mma32(a, b, acc); }
  static __device__ __forceinline__ Plain ld(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
  static constexpr bool kHasLo = true;
};
template <>
struct APolicy<float> {  // fp32 path
  using Split = f32x8;
  using Plain = f32x8;
  static __device__ __forceinline__ f32x8 split(const float* x) {
    return f32x8{x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  }
  static __device__ __forceinline__ f32x8 plain(const float* x) { return split(x); }
  static __device__ __forceinline__ f32x4 mma(const f32x8& a, const f32x8& b, f32x4 acc) { return mma32(a, b, acc); }
  static __device__ __forceinline__ f32x8 ld(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
  static constexpr bool kHasLo = false;
};

__device__ __forceinline__ int slot_row64(int p) { return (p & 32) + slot_row(p & 31); }

// LDS layout (bytes).  Small per-channel tables first, then the column
// factors of sub-tiles 0..2 (the only ones used as off-diagonal columns) and
// the fp32 UT inverse, row-major.
template <typename T, int D>
struct IntraLds {
  static constexpr int ES = sizeof(T);
  static constexpr int KP = D + 16 / ES;  // KC row pitch (elements)
  static constexpr int LP = 68;           // T row pitch (floats)
  static constexpr int LOC7 = 0;          // prefix at each sub-tile's anchor row  [4][D]
  static constexpr int TOT = LOC7 + 4 * D * 4;   // sub-tile totals              [4][D]
  static constexpr int ET = TOT + 4 * D * 4;     // e^{B_i - B_j}, 6 pairs i > j  [6][D]
  static constexpr int EB = ET + 6 * D * 4;      // e^{B_i}                       [4][D]
  static constexpr int EL = EB + 4 * D * 4;      // e^{G_last - B_i}              [4][D]
  static constexpr int BETA = EL + 4 * D * 4;    // beta                          [64]
  static constexpr int KC = BETA + 64 * 4;       // column factors                [48][KP]
  static constexpr int TM = KC + ((48 * KP * ES + 15) / 16) * 16;  // T          [64][LP]
  static constexpr int BYTES = TM + 64 * LP * 4;
};

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

template <typename T, int D>
__global__ __launch_bounds__(256, (sizeof(T) == 2 ? 3 : 2)) void kda_intra_kernel(const IntraParams p) {
  using L = IntraLds<T, D>;
  using AP = APolicy<T>;
  using R8 = Run8<T>;
  constexpr int KS = D / 32;
  constexpr int KP = L::KP, LP = L::LP;
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
  float* loc7 = reinterpret_cast<float*>(lds + L::LOC7);
  float* tot = reinterpret_cast<float*>(lds + L::TOT);
  float* Et = reinterpret_cast<float*>(lds + L::ET);
  float* eB = reinterpret_cast<float*>(lds + L::EB);
  float* eL = reinterpret_cast<float*>(lds + L::EL);
  float* betas = reinterpret_cast<float*>(lds + L::BETA);
  T* KC = reinterpret_cast<T*>(lds + L::KC);
  float* Tm = reinterpret_cast<float*>(lds + L::TM);

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int tok0 = p.t0 + c * kChunk;
  const int nvalid = min(kChunk, p.T - tok0);
  const int64_t tok_stride = (int64_t)p.H * D;
  const int64_t row0 = ((int64_t)b * p.T + tok0) * p.H * D + (int64_t)h * D;  // (token 0 of chunk, h)
  const int64_t rec = ((int64_t)b * p.H + h) * p.nc + c;
  constexpr RecLayout RL = rec_layout((int)sizeof(T), D);
  char* recp = p.ws.base + rec * p.ws.rec_bytes;
  T* qg = reinterpret_cast<T*>(recp + RL.qg);
  T* kg = reinterpret_cast<T*>(recp + RL.kg);
  T* kdt = reinterpret_cast<T*>(recp + RL.kdt);
  T* tb = reinterpret_cast<T*>(recp + RL.tb);
  T* aqh = reinterpret_cast<T*>(recp + RL.aqh);
  T* aql = reinterpret_cast<T*>(recp + RL.aql);
  float* gam = reinterpret_cast<float*>(recp + RL.gam);

  // ---- this wave's sub-tile rows of q, k, z (MFMA operand layout), beta ------
  const int ti = wave;
  const int r = 16 * ti + n;  // row of this lane in the chunk
  const bool rvalid = r < nvalid;
  typename R8::Raw qraw[KS], kraw[KS], zraw[KS];
  {
    const int64_t rowp = row0 + min(r, nvalid - 1) * tok_stride;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      qraw[kk] = R8::load(static_cast<const T*>(p.q) + rowp, kk, g4);
      kraw[kk] = R8::load(static_cast<const T*>(p.k) + rowp, kk, g4);
      zraw[kk] = R8::load(static_cast<const T*>(p.z) + rowp, kk, g4);
    }
  }
  const float beta_r =
      rvalid ? Elem<T>::to_f32(static_cast<const T*>(p.beta)[((int64_t)b * p.T + tok0 + r) * p.H + h]) : 0.0f;
  if (g4 == 0) betas[r] = beta_r;

  // ---- decay prefix within the sub-tile; anchor rows and totals to LDS --------
  float P[KS][8];
  subtile_decay_prefix<T, KS>(zraw, p.A[h], p.g_min, rvalid, P);
  if (n == 7)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) put_run8(loc7 + ti * D, kk, g4, P[kk]);
  if (n == 15)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) put_run8(tot + ti * D, kk, g4, P[kk]);
  const float nq = row_inv_norm<T, KS>(qraw, p.l2norm, p.l2_eps);
  const float nk = row_inv_norm<T, KS>(kraw, p.l2norm, p.l2_eps);
  const float rq = rvalid ? nq * p.q_scale : 0.0f;
  const float rk = rvalid ? nk : 0.0f;
  __syncthreads();

  // ---- per-channel tables from the sub-tile totals and anchors ---------------
  // G of sub-tile i = off_i + prefix, off_i = sum_{j < i} tot_j; B_i = off_i + loc7_i
  {
    constexpr int TPC = 256 / D;
    const int ch = tid % D, part = tid / D;
    float off[4], Bv[4];
    off[0] = 0.0f;
#pragma unroll
    for (int i = 1; i < 4; ++i) off[i] = off[i - 1] + tot[(i - 1) * D + ch];
    const float glast = off[3] + tot[3 * D + ch];
#pragma unroll
    for (int i = 0; i < 4; ++i) Bv[i] = off[i] + loc7[i * D + ch];
#pragma unroll
    for (int item = part; item < 15; item += TPC) {
      if (item < 4) {
        eB[item * D + ch] = hw_exp(Bv[item]);
      } else if (item < 8) {
        eL[(item - 4) * D + ch] = hw_exp(glast - Bv[item - 4]);
      } else if (item < 14) {
        const int pi = item - 8;  // pair index -> (i, j)
        const int i = (pi < 1) ? 1 : (pi < 3) ? 2 : 3;
        const int j = pi - pair_index(i, 0);
        Et[pi * D + ch] = hw_exp(Bv[i] - Bv[j]);
      } else {
        gam[ch] = hw_exp(glast);
      }
    }
  }
  __syncthreads();

  // ---- own sub-tile: factors, record rows, Kd^T, diagonal blocks -------------
  float KR[KS][8], QR[KS][8];  // row factors (kept for the off-diagonal blocks)
  f32x4 akk_d = zero4(), aqk_d = zero4();
  const typename AP::Plain sel0 = select_operand<typename AP::Plain>(n, g4, 0);
  const typename AP::Plain sel1 = select_operand<typename AP::Plain>(n, g4, 1);
  // record position of the four tokens 16 ti + 4 g4 + 0..3 inside a 64-token row
  const int tpos = 32 * (ti >> 1) + 8 * g4 + 4 * (ti & 1);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    float p7[8], eb[8], el[8];
    lds_run8(loc7 + ti * D, kk, g4, p7);
    lds_run8(eB + ti * D, kk, g4, eb);
    lds_run8(eL + ti * D, kk, g4, el);
    float kc[8], xq[8], xk[8], xd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float d = (P[kk][j] - p7[j]) * kLog2e;
      const float rf = hw_exp2(d);   // e^{G_r - B_i}
      const float cf = hw_exp2(-d);  // e^{B_i - G_r}
      const float qf = R8::get(qraw[kk], j);
      const float kf = R8::get(kraw[kk], j);
      KR[kk][j] = kf * (rk * rf);
      QR[kk][j] = qf * (rq * rf);
      kc[j] = kf * (rk * cf);
      xq[j] = QR[kk][j] * eb[j];  // q^ . Gamma
      xk[j] = -KR[kk][j] * eb[j];  // -(k^ . Gamma)
      xd[j] = kc[j] * el[j];      // k^ . Gamma_last / Gamma
    }
    store8<T>(qg + r * D + 32 * kk + 8 * g4, xq);
    store8<T>(kg + r * D + 32 * kk + 8 * g4, xk);
    if (ti < 3) store8<T>(KC + r * KP + 32 * kk + 8 * g4, kc);  // column factors for later sub-tiles
    {
      // lane (n, g4) receives Kd[16 ti + 4 g4 + i][32 kk + 16 half + n]
      const typename AP::Plain xdp = AP::plain(xd);
      const f32x4 t0 = AP::mma(xdp, sel0, zero4());
      const f32x4 t1 = AP::mma(xdp, sel1, zero4());
      store4<T>(kdt + (32 * kk + n) * kChunk + tpos, t0);
      store4<T>(kdt + (32 * kk + 16 + n) * kChunk + tpos, t1);
    }
    // transposed diagonal blocks: lane (n, g4) gets row n, columns 4 g4 + i
    akk_d = AP::mma(AP::plain(kc), AP::plain(KR[kk]), akk_d);
    aqk_d = AP::mma(AP::split(kc), AP::split(QR[kk]), aqk_d);
  }
  // L_ii = Diag(beta) StrictTril(A_kk(i, i)), staged where T_ii will go
  {
    f32x4 lv;
#pragma unroll
    for (int i = 0; i < 4; ++i) lv[i] = (4 * g4 + i < n) ? beta_r * akk_d[i] : 0.0f;
    *reinterpret_cast<f32x4*>(Tm + r * LP + 16 * ti + 4 * g4) = lv;
  }
  __syncthreads();  // column factors and the L_ii stages are visible

  // ---- off-diagonal blocks (ti, jt), jt < ti: plain products -----------------
  f32x4 akk[3], aqk[3];
#pragma unroll
  for (int jt = 0; jt < 3; ++jt) {
    akk[jt] = aqk[jt] = zero4();
    if (jt < ti) {
      const int pi = pair_index(ti, jt);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        float e8[8], xk[8], xq[8];
        lds_run8(Et + pi * D, kk, g4, e8);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xk[j] = KR[kk][j] * e8[j];
          xq[j] = QR[kk][j] * e8[j];
        }
        const typename AP::Plain aop = AP::ld(KC + (16 * jt + n) * KP + 32 * kk + 8 * g4);
        akk[jt] = AP::mma(aop, AP::plain(xk), akk[jt]);
        aqk[jt] = AP::mma(aop, AP::plain(xq), aqk[jt]);
      }
    }
  }

  // ---- Tril(A_qk) rows to the record (hi / lo), 8-byte stores ----------------
  // The scan reads the upper blocks (0, 1) and (2, 3) as part of its K-steps:
  // they are written as zeros.
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const bool lower = jt <= ti;
    const bool zero_blk = (ti == 0 && jt == 1) || (ti == 2 && jt == 3);
    if (lower || zero_blk) {
      f32x4 a;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = (jt == ti) ? ((4 * g4 + i <= n) ? aqk_d[i] : 0.0f) : (jt < ti ? aqk[jt < 3 ? jt : 0][i] : 0.0f);
        a[i] = v;
      }
      const int off = r * kChunk + 32 * (jt >> 1) + 8 * g4 + 4 * (jt & 1);
      store4<T>(aqh + off, a);
      if constexpr (AP::kHasLo) {
        f32x4 lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = a[i] - bf16_to_f32(f32_to_bf16(a[i]));
        store4<T>(aql + off, lo);
      }
    }
  }

  // ---- T_ii = (I + L_ii)^{-1}, row n, by back substitution over the columns --
  // T (I + L) = I gives T[n][c] = delta_nc - sum_{s > c} T[n][s] L[s][c]: once
  // T[n][s] is final its multiple of row s of L is removed from every column
  // c < s.  All four lane groups solve row n; group g4 keeps columns 4 g4 + i.
  f32x4 tii;
  {
    const float* Ls = Tm + (16 * ti) * LP + 16 * ti;
    float x[16];
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) x[cc] = (cc == n) ? 1.0f : 0.0f;
#pragma unroll
    for (int s = 15; s >= 1; --s) {
      float lrow[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        if (4 * q4 < s) {
          const float4 v = *reinterpret_cast<const float4*>(Ls + s * LP + 4 * q4);
          lrow[4 * q4] = v.x;
          lrow[4 * q4 + 1] = v.y;
          lrow[4 * q4 + 2] = v.z;
          lrow[4 * q4 + 3] = v.w;
        }
      }
      const float xs = x[s];
#pragma unroll
      for (int cc = 0; cc < s; ++cc) x[cc] -= xs * lrow[cc];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      tii[i] = (g4 == 0) ? x[i] : (g4 == 1) ? x[4 + i] : (g4 == 2) ? x[8 + i] : x[12 + i];
    __builtin_amdgcn_wave_barrier();  // every lane of the wave has read L_ii
    *reinterpret_cast<f32x4*>(Tm + r * LP + 16 * ti + 4 * g4) = tii;
  }
  // L rows of the off-diagonal blocks: A operands of the level products
#pragma unroll
  for (int jt = 0; jt < 3; ++jt)
#pragma unroll
    for (int i = 0; i < 4; ++i) akk[jt][i] *= beta_r;
  __syncthreads();  // every T_ii is in LDS

  // ---- off-diagonal blocks of T by distance: T_ij = -T_ii sum_{m=j}^{i-1} L_im T_mj
  // fp32 MFMA 16x16x4 with K index 4 g + t in step t: the A operands are the
  // rows this lane holds (L_im, T_ii), the B operands columns (T_mj from LDS,
  // and the accumulator P as produced).
#pragma unroll
  for (int dist = 1; dist <= 3; ++dist) {
    if (ti >= dist) {
      const int j = ti - dist;
      f32x4 Pm = zero4();
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        if (m >= j && m < ti) {
#pragma unroll
          for (int t = 0; t < 4; ++t) Pm = mfma4(akk[m][t], Tm[(16 * m + 4 * g4 + t) * LP + 16 * j + n], Pm);
        }
      }
      f32x4 Tn = zero4();
#pragma unroll
      for (int t = 0; t < 4; ++t) Tn = mfma4(tii[t], Pm[t], Tn);
      // lane holds column 16 j + n, rows 16 ti + 4 g4 + i
#pragma unroll
      for (int i = 0; i < 4; ++i) Tm[(16 * ti + 4 * g4 + i) * LP + 16 * j + n] = -Tn[i];
    }
    __syncthreads();
  }

  // ---- tb = T Diag(beta), columns in slot order; upper blocks are zero -------
  for (int idx = tid; idx < kChunk * 8; idx += 256) {
    const int rr = idx >> 3, pg = idx & 7;
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = slot_row64(8 * pg + j);
      x[j] = ((s >> 4) <= (rr >> 4)) ? Tm[rr * LP + s] * betas[s] : 0.0f;
    }
    store8<T>(tb + rr * kChunk + 8 * pg, x);
  }
}

hipError_t launch_intra(const IntraParams& p, int D, int in_f32, hipStream_t s) {
  const dim3 grid(p.nc, p.H, p.B), block(256);
  if (in_f32) {
    if (D == 64) hipLaunchKernelGGL((kda_intra_kernel<float, 64>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((kda_intra_kernel<float, 128>), grid, block, 0, s, p);
  } else {
    if (D == 64) hipLaunchKernelGGL((kda_intra_kernel<uint16_t, 64>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((kda_intra_kernel<uint16_t, 128>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kda
