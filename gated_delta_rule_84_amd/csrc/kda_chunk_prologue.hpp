// Chunk prologue shared by the intra-chunk kernel and the pre-pass kernel:
// the K3 bounded log-decay of a 64-token chunk, its chunk-local inclusive
// cumulative sum, and the q / k inverse L2 norms of one 16-token sub-tile.
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3), section 2.1 (L2Norm on q and k) and
// section 2.2 (g = g_min * Sigmoid(e^{A_h} z), alpha = e^g; Gamma is the
// cumulative product of retentions, kept here as its logarithm G).
#pragma once

#include "kda_common.hpp"
#include "kda_params.hpp"

namespace kda {

// Channel set of a lane in one 32-wide K-step: lane group g owns positions
// 8 g .. 8 g + 7 of the step, which hold channels 32 kk + slot_row(8 g + j),
// i.e. the two runs 32 kk + 4 g + 0..3 and 32 kk + 16 + 4 g + 0..3.
__device__ __forceinline__ int lane_ch(int kk, int g, int j) { return 32 * kk + 16 * (j >> 2) + 4 * g + (j & 3); }

// 8 elements of a row in a lane's channel set, as a raw MFMA operand.
template <typename T>
struct Run8;
template <>
struct Run8<uint16_t> {
  using Raw = bf16x8;
  static __device__ __forceinline__ Raw load(const uint16_t* row, int kk, int g) {
    const uint2 a = *reinterpret_cast<const uint2*>(row + 32 * kk + 4 * g);
    const uint2 b = *reinterpret_cast<const uint2*>(row + 32 * kk + 16 + 4 * g);
    const u32x4 w = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, w);
  }
  static __device__ __forceinline__ float get(const Raw& r, int j) { return static_cast<float>(r[j]); }
};
template <>
struct Run8<float> {
  using Raw = f32x8;
  static __device__ __forceinline__ Raw load(const float* row, int kk, int g) {
    const float4 a = *reinterpret_cast<const float4*>(row + 32 * kk + 4 * g);
    const float4 b = *reinterpret_cast<const float4*>(row + 32 * kk + 16 + 4 * g);
    return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
  static __device__ __forceinline__ float get(const Raw& r, int j) { return r[j]; }
};

// 8 fp32 of a row in a lane's channel set, from an LDS row (two float4 reads).
__device__ __forceinline__ void lds_run8(const float* row, int kk, int g, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(row + 32 * kk + 4 * g);
  const float4 b = *reinterpret_cast<const float4*>(row + 32 * kk + 16 + 4 * g);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
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

// 256 threads.  G[64][D + 4] (LDS, fp32) receives, per channel, the
// inclusive cumulative sum over the chunk's tokens of
//     g = g_min * Sigmoid(e^{A_h} z)      (0 for rows r >= nvalid),
// summed as per-segment prefixes plus the totals of the earlier segments
// (256 / D segments per channel).  tot needs 256 floats.  Ends after a
// barrier with G complete.  zrow0 points at (token 0 of the chunk, head h,
// channel 0); tokens are tok_stride elements apart.
template <typename T, int D>
__device__ __forceinline__ void decay_cumsum(float* G, float* tot, const T* __restrict__ zrow0, int64_t tok_stride,
                                             int nvalid, float A_h, float g_min) {
  constexpr int GP = D + 4;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int VPR = D / VEC;
  constexpr int TPC = 256 / D;   // threads per channel
  constexpr int RPS = 64 / TPC;  // rows per segment
  const int tid = threadIdx.x;
  const float eA = hw_exp(A_h);
#pragma unroll
  for (int it = 0; it < (64 * VPR) / 256; ++it) {
    const int idx = tid + 256 * it;
    const int r = idx / VPR;
    const int cv = (idx % VPR) * VEC;
    const u32x4 raw = *reinterpret_cast<const u32x4*>(zrow0 + min(r, nvalid - 1) * tok_stride + cv);
    const T* zt = reinterpret_cast<const T*>(&raw);
    float gv[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) gv[e] = (r < nvalid) ? g_min * sigmoid_fast(eA * Elem<T>::to_f32(zt[e])) : 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; e += 4)
      *reinterpret_cast<float4*>(&G[r * GP + cv + e]) = make_float4(gv[e], gv[e + 1], gv[e + 2], gv[e + 3]);
  }
  __syncthreads();
  const int ch = tid % D, seg = tid / D;
  float acc[RPS];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < RPS; ++i) {
    s += G[(seg * RPS + i) * GP + ch];
    acc[i] = s;
  }
  tot[seg * D + ch] = s;
  __syncthreads();
  float off = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < TPC - 1; ++s2)
    if (s2 < seg) off += tot[s2 * D + ch];
#pragma unroll
  for (int i = 0; i < RPS; ++i) G[(seg * RPS + i) * GP + ch] = acc[i] + off;
  __syncthreads();
}

// Inverse L2 norm of the lane's row (row n of a 16-row sub-tile) from the
// diagonal of X X^T on MFMA (bf16 products are exact in fp32; sums in fp32).
// x[kk] is the lane's raw operand of K-step kk; every lane of the row gets
// 1 / sqrt(|x|^2 + eps) (1 when l2norm == 0).
template <typename T, int KS>
__device__ __forceinline__ float row_inv_norm(const typename Run8<T>::Raw* x, int l2norm, float eps) {
  const int lane = threadIdx.x & 63, n = lane & 15;
  f32x4 acc = zero4();
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) acc = mma32(x[kk], x[kk], acc);
  // lane (n, g) holds rows 4 g .. 4 g + 3 of column n: the diagonal entry of
  // row n sits in lane (n, n / 4) at index n % 4
  const int i = n & 3;
  const float d = (i == 0) ? acc[0] : (i == 1) ? acc[1] : (i == 2) ? acc[2] : acc[3];
  const float dn = __shfl(d, n + 16 * (n >> 2));
  return l2norm ? hw_rsqrt(dn + eps) : 1.0f;
}

}  // namespace kda
