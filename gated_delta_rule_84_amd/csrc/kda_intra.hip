// Intra-chunk kernel: everything of a 64-token chunk that does not depend on
// the recurrent state.  One workgroup (4 waves) per (chunk, head, batch).
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3).  Section 2.1 gives the chunked output
// O = (Gamma . Q) S + Tril[(Q . Gamma)(K / Gamma)^T](U - W S); U and W are the
// UT-transform pair (I + StrictTril(Diag(beta)(K . Gamma)(K / Gamma)^T))^{-1}
// applied to Diag(beta) V and Diag(beta)(K . Gamma).  Section 2.2: the chunk is
// cut into 16-token sub-tiles and, because the K3 decay keeps a sub-tile's
// cumulative log-decay within (-80, 0), every causal sub-tile block --
// diagonal blocks included -- is a dense matrix product of decay-scaled
// factors.  Here each row sub-tile i is anchored at its 8th token,
// Bi = G[16 i + 7], so both factors of every block stay within e^{+-40}:
//     A(i, j) = (K_i . e^{G_i - Bi}) (K_j . e^{Bi - G_j})^T.
// The A products use bf16 MFMA on hi/lo split operands (three products per
// step) because a plain bf16 product misses the output tolerance; the fp32
// path uses fp32 MFMA.
//
// Outputs (one ChunkWs record per chunk):
//   qg = q^ . Gamma, kg = k^ . Gamma, kdt = (k^ . Gamma_last / Gamma)^T,
//   tb = T Diag(beta) with T = (I + Diag(beta) StrictTril(A_kk))^{-1},
//   aq = Tril(A_qk) (diagonal included), gam = Gamma_last.
#include "kda_chunk_prologue.hpp"

namespace kda {

template <typename T>
struct APolicy;
template <>
struct APolicy<uint16_t> {  // bf16 path: split operands, three MFMAs per step
  struct Op {
    bf16x8 hi, lo;
  };
  static __device__ __forceinline__ Op make(const float* x) {
    Op o;
    split8_bf16(x, o.hi, o.lo);
    return o;
  }
  static __device__ __forceinline__ f32x4 mma(const Op& a, const Op& b, f32x4 acc) {
    return mma32_x3(a.hi, a.lo, b.hi, b.lo, acc);
  }
};
template <>
struct APolicy<float> {
  struct Op {
    f32x8 v;
  };
  static __device__ __forceinline__ Op make(const float* x) {
    Op o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o.v[j] = x[j];
    return o;
  }
  static __device__ __forceinline__ f32x4 mma(const Op& a, const Op& b, f32x4 acc) {
    return mma32(a.v, b.v, acc);
  }
};

__device__ __forceinline__ int slot_pos64(int s) { return (s & 32) + slot_pos(s & 31); }
__device__ __forceinline__ int slot_row64(int p) { return (p & 32) + slot_row(p & 31); }

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void kda_intra_kernel(const IntraParams p) {
  __shared__ ChunkSmem<T, D> sm;
  constexpr int GP = ChunkSmem<T, D>::GP;
  constexpr int XP = ChunkSmem<T, D>::XP;
  constexpr int LP = ChunkSmem<T, D>::LP;
  using AP = APolicy<T>;

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok0 = p.t0 + c * kChunk;
  const int nvalid = min(kChunk, p.T - tok0);
  const int64_t rec = ((int64_t)b * p.H + h) * p.nc + c;

  chunk_prologue<T, D>(sm, static_cast<const T*>(p.q), static_cast<const T*>(p.k),
                       static_cast<const T*>(p.z), static_cast<const T*>(p.beta), p.A[h], b, h, p.T,
                       p.H, tok0, nvalid, p.g_min, p.l2_eps, p.l2norm);

  constexpr RecLayout RL = rec_layout((int)sizeof(T), D);
  char* recp = p.ws.base + rec * p.ws.rec_bytes;
  T* qg = reinterpret_cast<T*>(recp + RL.qg);
  T* kg = reinterpret_cast<T*>(recp + RL.kg);
  T* kdt = reinterpret_cast<T*>(recp + RL.kdt);
  T* tb = reinterpret_cast<T*>(recp + RL.tb);
  T* aqh = reinterpret_cast<T*>(recp + RL.aqh);
  T* aql = reinterpret_cast<T*>(recp + RL.aql);
  float* gam = reinterpret_cast<float*>(recp + RL.gam);
  const float* G = sm.u0.G;

  // ---- factor tensors for the state scan (columns in slot order) ----------
  for (int idx = tid; idx < kChunk * (D / 8); idx += 256) {
    const int r = idx / (D / 8), pg = idx % (D / 8);
    const int cb = 32 * (pg >> 2);
    float xq[8], xk[8];
    const float sq = sm.rq[r] * p.q_scale, sk = sm.rk[r];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ch = cb + slot_row(8 * (pg & 3) + j);
      const float e = hw_exp2(G[r * GP + ch] * kLog2e);
      xq[j] = Elem<T>::to_f32(sm.u1.x.q[r * XP + ch]) * sq * e;
      xk[j] = Elem<T>::to_f32(sm.u1.x.k[r * XP + ch]) * sk * e;
    }
    store8<T>(qg + r * D + 8 * pg, xq);
    store8<T>(kg + r * D + 8 * pg, xk);
  }
  for (int idx = tid; idx < D * 8; idx += 256) {
    const int ch = idx >> 3, pg = idx & 7;  // 8 neighbouring threads fill one kdt row
    const float glast = G[(kChunk - 1) * GP + ch];
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = slot_row64(8 * pg + j);
      x[j] = Elem<T>::to_f32(sm.u1.x.k[r * XP + ch]) * sm.rk[r] * hw_exp2((glast - G[r * GP + ch]) * kLog2e);
    }
    store8<T>(kdt + ch * kChunk + 8 * pg, x);
  }
  if (tid < D) gam[tid] = hw_exp2(G[(kChunk - 1) * GP + tid] * kLog2e);

  // ---- sub-tile products A_kk(i, j), A_qk(i, j), j <= i; wave i = row tile --
  const int n = lane & 15, g4 = lane >> 4;
  const int ti = wave;
  const int r = 16 * ti + n;
  const int ra = 16 * ti + 7;  // anchor row of this row tile
  f32x4 akk[4], aqk[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) akk[jt] = aqk[jt] = zero4();
  {
    const float sq = sm.rq[r] * p.q_scale, sk = sm.rk[r];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const int c0 = 32 * kk + 8 * g4;
      float gr[8], ga[8], xq[8], xk[8];
      load8_lds<float>(&G[r * GP + c0], gr);
      load8_lds<float>(&G[ra * GP + c0], ga);
      load8_lds<T>(&sm.u1.x.q[r * XP + c0], xq);
      load8_lds<T>(&sm.u1.x.k[r * XP + c0], xk);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float e = hw_exp2((gr[j] - ga[j]) * kLog2e);
        xq[j] *= sq * e;
        xk[j] *= sk * e;
      }
      const typename AP::Op oq = AP::make(xq), ok = AP::make(xk);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (jt <= ti) {
          const int s = 16 * jt + n;
          float gs[8], y[8];
          load8_lds<float>(&G[s * GP + c0], gs);
          load8_lds<T>(&sm.u1.x.k[s * XP + c0], y);
          const float ss = sm.rk[s];
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] *= ss * hw_exp2((ga[j] - gs[j]) * kLog2e);
          const typename AP::Op oy = AP::make(y);
          akk[jt] = AP::mma(ok, oy, akk[jt]);
          aqk[jt] = AP::mma(oq, oy, aqk[jt]);
        }
      }
    }
  }
  __syncthreads();  // q, k, G no longer read: their LDS becomes L and Tm

  // L = Diag(beta) StrictTril(A_kk) into LDS; Tril(A_qk) staged in LDS (slot
  // order) for coalesced stores of its hi / lo parts.
  float* Aq = sm.u0.Tm;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int rr = 16 * ti + 4 * g4 + ii;
      const int s = 16 * jt + n;
      const float vkk = (jt <= ti && s < rr) ? sm.beta[rr] * akk[jt][ii] : 0.0f;
      const float vqk = (jt <= ti && s <= rr) ? aqk[jt][ii] : 0.0f;
      sm.u1.L[rr * LP + s] = vkk;
      Aq[rr * LP + slot_pos64(s)] = vqk;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < kChunk * 8; idx += 256) {
    const int rr = idx >> 3, pg = idx & 7;
    float x[8], lo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = Aq[rr * LP + 8 * pg + j];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) lo[j] = x[j] - bf16_to_f32(f32_to_bf16(x[j]));
      store8<T>(aql + rr * kChunk + 8 * pg, lo);
    }
    store8<T>(aqh + rr * kChunk + 8 * pg, x);
  }
  __syncthreads();

  // ---- T = (I + L)^{-1}: diagonal 16x16 blocks by forward substitution ------
  float* Tm = sm.u0.Tm;
  const float* L = sm.u1.L;
  if (wave == 0) {
    const int ib = lane >> 4, col = lane & 15;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float acc = (rr == col) ? 1.0f : 0.0f;
#pragma unroll
      for (int ss = 0; ss < rr; ++ss) acc -= L[(16 * ib + rr) * LP + 16 * ib + ss] * x[ss];
      x[rr] = acc;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) Tm[(16 * ib + rr) * LP + 16 * ib + col] = x[rr];
  } else {
    // zero the strictly-upper blocks
    for (int idx = tid - 64; idx < 6 * 256; idx += 192) {
      const int blk = idx >> 8, e = idx & 255;
      const int bi = (blk < 3) ? 0 : (blk < 5 ? 1 : 2);
      const int bj = (blk < 3) ? blk + 1 : (blk < 5 ? blk - 1 : 3);
      Tm[(16 * bi + (e >> 4)) * LP + 16 * bj + (e & 15)] = 0.0f;
    }
  }
  __syncthreads();
  // off-diagonal blocks by distance: T_ij = -T_ii * sum_{m=j}^{i-1} L_im T_mj
  {
    const int pr = lane >> 2, pc = (lane & 3) * 4;
#pragma unroll
    for (int dist = 1; dist <= 3; ++dist) {
      const int bj = wave, bi = wave + dist;
      const bool active = (bi <= 3);
      if (active) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int bm = bj; bm < bi; ++bm) {
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            const float l = L[(16 * bi + pr) * LP + 16 * bm + m];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += l * Tm[(16 * bm + m) * LP + 16 * bj + pc + e];
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.P[wave][pr * 17 + pc + e] = acc[e];
      }
      __syncthreads();
      if (active) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          const float t = Tm[(16 * bi + pr) * LP + 16 * bi + m];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += t * sm.P[wave][m * 17 + pc + e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) Tm[(16 * bi + pr) * LP + 16 * bj + pc + e] = -acc[e];
      }
      __syncthreads();
    }
  }

  // tb = T Diag(beta), columns in slot order
  for (int idx = tid; idx < kChunk * 8; idx += 256) {
    const int rr = idx >> 3, pg = idx & 7;
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = slot_row64(8 * pg + j);
      x[j] = Tm[rr * LP + s] * sm.beta[s];
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
