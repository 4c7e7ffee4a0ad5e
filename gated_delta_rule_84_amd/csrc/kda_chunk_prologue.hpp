// Chunk prologue shared by the intra-chunk kernel and the pre-pass kernel:
// loads one 64-token chunk of one head into LDS and computes the K3 bounded
// log-decay, its chunk-local inclusive cumulative sum and the q / k inverse
// L2 norms.
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3), section 2.1 (L2Norm on q and k) and
// section 2.2 (g = g_min * Sigmoid(e^{A_h} z), alpha = e^g; Gamma is the
// cumulative product of retentions, kept here as its logarithm G).
#pragma once

#include "kda_common.hpp"
#include "kda_params.hpp"

namespace kda {

template <typename T, int D>
struct ChunkSmem {
  static constexpr int GP = D + 4;                  // fp32 row pitch of G (bank spread)
  static constexpr int XP = D + 16 / (int)sizeof(T);  // row pitch of q / k (+16 bytes)
  static constexpr int LP = 64 + 4;                 // fp32 row pitch of 64x64 matrices
  union {
    float G[kChunk * GP];   // cumulative log-decay, later the UT inverse (pitch LP)
    float Tm[kChunk * LP];
  } u0;
  union {
    struct {
      T q[kChunk * XP];
      T k[kChunk * XP];
    } x;
    float L[kChunk * LP];   // Diag(beta) StrictTril(A_kk), after the products
  } u1;
  float rq[kChunk];
  float rk[kChunk];
  float beta[kChunk];
  float P[3][16 * 17];      // scratch for the block inverse
};

template <typename T>
__device__ __forceinline__ void load8_lds(const T* p, float* out);
template <>
__device__ __forceinline__ void load8_lds<uint16_t>(const uint16_t* p, float* out) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8_lds<float>(const float* p, float* out) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// Store 8 fp32 values as 8 elements of T (16 or 32 bytes, aligned).
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* x);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float* x) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(f32_to_bf16(x[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(x[2 * i + 1])) << 16);
  *reinterpret_cast<u32x4*>(p) = w;
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// 256 threads.  After return (and its trailing barrier) the LDS holds, for the
// chunk's rows r < nvalid (zeros / flat decay beyond):
//   x.q, x.k : raw q, k;   rq, rk : inverse L2 norms (1 when l2norm == 0)
//   G        : inclusive cumulative sum of g over the chunk, per channel
//   beta     : beta (0 beyond nvalid, or everywhere when beta is null)
template <typename T, int D>
__device__ __forceinline__ void chunk_prologue(ChunkSmem<T, D>& sm, const T* __restrict__ q,
                                               const T* __restrict__ k, const T* __restrict__ z,
                                               const T* __restrict__ beta, float A_h, int b, int h,
                                               int T_total, int H, int tok0, int nvalid, float g_min,
                                               float l2_eps, int l2norm) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int VPR = D / VEC;
  constexpr int GP = ChunkSmem<T, D>::GP;
  constexpr int XP = ChunkSmem<T, D>::XP;
  const int tid = threadIdx.x;
  const float eA = hw_exp2(A_h * kLog2e);
  for (int idx = tid; idx < kChunk * VPR; idx += 256) {
    const int r = idx / VPR;
    const int cv = (idx % VPR) * VEC;
    u32x4 vq = {0u, 0u, 0u, 0u}, vk = {0u, 0u, 0u, 0u}, vz = {0u, 0u, 0u, 0u};
    if (r < nvalid) {
      const int64_t off = ((int64_t)(b * (int64_t)T_total + tok0 + r) * H + h) * D + cv;
      vq = *reinterpret_cast<const u32x4*>(q + off);
      vk = *reinterpret_cast<const u32x4*>(k + off);
      vz = *reinterpret_cast<const u32x4*>(z + off);
    }
    *reinterpret_cast<u32x4*>(&sm.u1.x.q[r * XP + cv]) = vq;
    *reinterpret_cast<u32x4*>(&sm.u1.x.k[r * XP + cv]) = vk;
    float zf[VEC];
    const T* zt = reinterpret_cast<const T*>(&vz);
#pragma unroll
    for (int e = 0; e < VEC; ++e) zf[e] = Elem<T>::to_f32(zt[e]);
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      sm.u0.G[r * GP + cv + e] = (r < nvalid) ? g_min * sigmoid_fast(eA * zf[e]) : 0.0f;
  }
  if (tid < kChunk) {
    float bv = 0.f;
    if (tid < nvalid && beta != nullptr) bv = Elem<T>::to_f32(beta[(int64_t)(b * (int64_t)T_total + tok0 + tid) * H + h]);
    sm.beta[tid] = bv;
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll 8
    for (int r = 0; r < kChunk; ++r) {
      s += sm.u0.G[r * GP + tid];
      sm.u0.G[r * GP + tid] = s;
    }
  } else if (tid < D + 2 * kChunk) {
    const int r = (tid - D) & (kChunk - 1);
    const T* row = (tid - D < kChunk) ? &sm.u1.x.q[r * XP] : &sm.u1.x.k[r * XP];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < D; c += 8) {
      float x[8];
      load8_lds<T>(row + c, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
    }
    const float rn = l2norm ? hw_rsqrt(ss + l2_eps) : 1.0f;
    if (tid - D < kChunk)
      sm.rq[r] = rn;
    else
      sm.rk[r] = rn;
  }
  __syncthreads();
}

}  // namespace kda
