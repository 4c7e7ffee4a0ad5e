// Chunk prologue shared by the intra-chunk kernel and the pre-pass kernel.
// One wave owns one 16-token sub-tile; lane (n, g) holds row n of the
// sub-tile at the channels of its MFMA operand slots.  From those rows it
// forms the K3 bounded log-decay, its inclusive prefix within the sub-tile
// (across the 16 lanes of a row group, in registers) and the q / k inverse
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

// 8 fp32 of a channel-indexed row in a lane's channel set (two float4 reads).
__device__ __forceinline__ void lds_run8(const float* row, int kk, int g, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(row + 32 * kk + 4 * g);
  const float4 b = *reinterpret_cast<const float4*>(row + 32 * kk + 16 + 4 * g);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
// ... and the inverse: write a lane's 8 channel values into a channel-indexed row.
__device__ __forceinline__ void put_run8(float* row, int kk, int g, const float* x) {
  *reinterpret_cast<float4*>(row + 32 * kk + 4 * g) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(row + 32 * kk + 16 + 4 * g) = make_float4(x[4], x[5], x[6], x[7]);
}

// Store 8 fp32 values as 8 elements of T (16 or 32 bytes, aligned).
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* x);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float* x) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = pack2_bf16(x[2 * i], x[2 * i + 1]);
  *reinterpret_cast<u32x4*>(p) = w;
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// Store 4 fp32 values as 4 elements of T (8 or 16 bytes, aligned).
template <typename T>
__device__ __forceinline__ void store4(T* p, const f32x4& x);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, const f32x4& x) {
  uint2 w;
  w.x = pack2_bf16(x[0], x[1]);
  w.y = pack2_bf16(x[2], x[3]);
  *reinterpret_cast<uint2*>(p) = w;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const f32x4& x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// x + (value of the lane S places below in the same 16-lane row; 0 past the
// row's start): one step of an inclusive prefix sum across a row group.
template <int S>
__device__ __forceinline__ float add_row_shr(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + S, 0xf, 0xf, true);
  return x + __builtin_bit_cast(float, y);
}

// Decay of this lane's row and channels, and its inclusive prefix over the
// sub-tile's rows 0..n (lanes n of the lane's row group):
//     P[kk][j] = sum_{m <= n} g(m, lane_ch(kk, g, j)) * unit
// with the K3 map g = g_min Sigmoid(e^{A_h} z) (section 2.2) or, with
// SOFTPLUS, Kimi Linear's g = -e^{A_h} Softplus(z) (the map section 2.2
// replaces; unbounded below).  unit = 1 gives the log-decay prefix G,
// unit = log2(e) gives G in base-2 units, ready for exp2.  Rows past the end
// of the sequence (valid == false) contribute 0.
template <typename T, int KS, bool SOFTPLUS = false>
__device__ __forceinline__ void subtile_decay_prefix(const typename Run8<T>::Raw* z, float A_h, float g_min,
                                                     float unit, bool valid, float (&P)[KS][8]) {
  const float eA = hw_exp(A_h);
  const float c1 = -eA * kLog2e;                            // Sigmoid(e^A z) = 1 / (1 + 2^{c1 z})
  const float gm = valid ? g_min * unit : 0.0f;             // K3 scale
  const float sp = valid ? -eA * unit * (1.0f / kLog2e) : 0.0f;  // softplus scale (softplus_log2 is in base 2)
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x;
      if constexpr (SOFTPLUS)
        x = sp * softplus_log2(Run8<T>::get(z[kk], j));
      else
        x = gm * hw_rcp(1.0f + hw_exp2(c1 * Run8<T>::get(z[kk], j)));
      x = add_row_shr<1>(x);
      x = add_row_shr<2>(x);
      x = add_row_shr<4>(x);
      x = add_row_shr<8>(x);
      P[kk][j] = x;
    }
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
