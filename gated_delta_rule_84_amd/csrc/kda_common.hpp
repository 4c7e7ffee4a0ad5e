// Shared device helpers for the KDA kernels (gfx950 / CDNA4, wave64).
//
// MFMA conventions used throughout (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32, lane l, lane group g = l / 16, n = l % 16):
//   A operand (16 x K): lane holds row n, 8 K-slots of group g
//   B operand (K x 16): lane holds column n, the same 8 K-slots of group g
//   C / D     (16 x 16): lane holds rows 4g .. 4g+3 of column n
// A contraction may visit its K index in any order as long as A and B agree,
// so every "K-step" of 32 handled by one lane-group slot pattern is written
// as 8 values per lane.  When an accumulator (C layout, rows on M) has to
// feed the next product as its B operand (rows on K), the K-slots of a step
// are mapped onto the rows the lane already holds:
//   slot j of group g in step kk  <->  row 32*kk + 16*(j / 4) + 4*g + (j % 4)
// and the matching A operand is stored with its columns in that order
// ("slot order"), so it is still one contiguous 8-element load per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr float kLog2e = 1.4426950408889634f;

// Position p (0..31) inside a 32-wide step holds logical index slot_row(p).
__host__ __device__ constexpr int slot_row(int p) {
  return 16 * ((p & 7) >> 2) + 4 * (p >> 3) + (p & 3);
}
// Inverse: logical index s (0..31) sits at position slot_pos(s).
__host__ __device__ constexpr int slot_pos(int s) {
  return 8 * ((s & 15) >> 2) + 4 * (s >> 4) + (s & 3);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// ---- element types of the two precision policies -------------------------
// bf16 path: bf16 inputs, bf16 MFMA operands, hi/lo split where needed.
// f32 path : fp32 inputs, fp32 MFMA operands throughout.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {  // bf16 storage
  using vec8 = bf16x8;
  static __device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
  static __device__ __forceinline__ uint16_t from_f32(float x) { return f32_to_bf16(x); }
};
template <> struct Elem<float> {
  using vec8 = f32x8;
  static __device__ __forceinline__ float to_f32(float x) { return x; }
  static __device__ __forceinline__ float from_f32(float x) { return x; }
};

// 8 fp32 -> packed operand of the given element type.
__device__ __forceinline__ bf16x8 pack8_bf16(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = static_cast<__bf16>(x[j]);
  return r;
}
// hi = bf16(x), lo = bf16(x - hi): x ~= hi + lo to about 16 bits.
__device__ __forceinline__ void split8_bf16(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    __bf16 h = static_cast<__bf16>(x[j]);
    hi[j] = h;
    lo[j] = static_cast<__bf16>(x[j] - static_cast<float>(h));
  }
}

// ---- one K=32 step: acc += A(16x32) * B(32x16) ---------------------------
__device__ __forceinline__ f32x4 mma32(const bf16x8& a, const bf16x8& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(const f32x8& a, const f32x8& b, f32x4 acc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
  return acc;
}
// Three-term split product: (ah + al)(bh + bl) without the al*bl term.
__device__ __forceinline__ f32x4 mma32_x3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                          const bf16x8& bl, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}

// Accumulator pair (rows 4g..4g+3 of two 16-row tiles) -> B operand in slot
// order.
__device__ __forceinline__ bf16x8 acc_pair_to_bf16(const f32x4& t0, const f32x4& t1) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = static_cast<__bf16>(t0[i]);
    r[4 + i] = static_cast<__bf16>(t1[i]);
  }
  return r;
}
__device__ __forceinline__ void acc_pair_split(const f32x4& t0, const f32x4& t1, bf16x8& hi, bf16x8& lo) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = t0[i];
    x[4 + i] = t1[i];
  }
  split8_bf16(x, hi, lo);
}
__device__ __forceinline__ f32x8 acc_pair_to_f32(const f32x4& t0, const f32x4& t1) {
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = t0[i];
    r[4 + i] = t1[i];
  }
  return r;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Hardware transcendental approximations (about 1 ulp): 2^x, 1/x and
// 1/sqrt(x).  2^x flushes results below the normal range to 0, which is the
// right limit everywhere they are used here (decay factors and gates whose
// true values are negligibly small).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float hw_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float hw_exp(float x) { return hw_exp2(x * kLog2e); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// Softplus(x) log2(e) = log2(1 + e^x) = max(x, 0) log2(e) + log2(1 + 2^{-|x| log2(e)}).
// Where 1 + e^{-|x|} rounds to 1 the last term is below fp32 resolution of
// the result (or the decay it feeds is 1 to fp32 accuracy).
__device__ __forceinline__ float softplus_log2(float x) {
  return fmaxf(x, 0.0f) * kLog2e + hw_log2(1.0f + hw_exp2(-fabsf(x) * kLog2e));
}

// Logistic function: 1 / (1 + e^{-x}); saturates to 0 and 1 at the extremes.
__device__ __forceinline__ float sigmoid_fast(float x) { return hw_rcp(1.0f + hw_exp2(-x * kLog2e)); }

}  // namespace kda
