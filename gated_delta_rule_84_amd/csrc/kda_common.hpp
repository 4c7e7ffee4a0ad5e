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
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

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
// Two fp32 values as packed bf16 (a in the low half), one v_cvt_pk_bf16_f32
// with both sources (the same rounding as f32_to_bf16; converting element
// by element instead packs each value alone and merges them with two more
// instructions).
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
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
  const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, bf16x8);  // four paired conversions
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
__device__ __forceinline__ f32x4 mma32(const f16x8& a, const f16x8& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}

// Accumulator pair (rows 4g..4g+3 of two 16-row tiles) -> B operand in slot
// order.
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

// ---- precision of the chunk record and of the state scan's products --------
// bf16 inputs: the record entries, the state and the residuals enter the
// scan's products as fp16 (11-bit significands, round to nearest even,
// v_cvt_pk_f16_f32), accumulated in fp32.  Every record entry is bounded:
// |q^ . Gamma|, |k^ . Gamma|, |Kd| <= 1 (unit rows, retentions <= 1),
// |Tril(A_qk)| <= 1 and |T Diag(beta)| <= 1 (the UT transform maps each value
// row to the delta-rule update of a state built from the chunk's own earlier
// rows, whose norm the unit keys and beta <= 1 bound).  The state itself is
// unbounded in principle, so it is held scaled by a power of two, S * 2^-4:
// q^ . Gamma and k^ . Gamma are stored times 2^4 and Kd times 2^-4, which
// leaves every product unchanged and lets |S| reach ~1e6 before its fp16
// copy overflows.  fp32 inputs: fp32 everywhere, no scaling.
template <typename T>
struct RecOps;
template <>
struct RecOps<uint16_t> {  // bf16 inputs
  using Elem = uint16_t;   // fp16 bits
  using V8 = f16x8;
  static constexpr float kLog2Up = 4.0f;        // log2 of the factor on q^ . Gamma and k^ . Gamma
  static constexpr float kStateScale = 0.0625f;  // the state is held as S * 2^-4
  static __device__ __forceinline__ V8 plain(const float* x) {
    V8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = static_cast<_Float16>(x[j]);
    return r;
  }
  static __device__ __forceinline__ V8 plain_acc(const f32x4& a, const f32x4& b) {
    V8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = static_cast<_Float16>(a[i]);
      r[4 + i] = static_cast<_Float16>(b[i]);
    }
    return r;
  }
  // 8 values as 16 bytes (one record unit)
  static __device__ __forceinline__ u32x4 pack8(const float* x) { return __builtin_bit_cast(u32x4, plain(x)); }
  // 4 values as 8 bytes
  static __device__ __forceinline__ uint2 pack4(const f32x4& x) {
    f16x4 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = static_cast<_Float16>(x[i]);
    return __builtin_bit_cast(uint2, h);
  }
  static __device__ __forceinline__ f32x4 mma(const V8& a, const V8& b, f32x4 acc) { return mma32(a, b, acc); }
};
template <>
struct RecOps<float> {  // fp32 inputs
  using Elem = float;
  using V8 = f32x8;
  static constexpr float kLog2Up = 0.0f;
  static constexpr float kStateScale = 1.0f;
  static __device__ __forceinline__ V8 plain(const float* x) {
    return f32x8{x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  }
  static __device__ __forceinline__ V8 plain_acc(const f32x4& a, const f32x4& b) { return acc_pair_to_f32(a, b); }
  static __device__ __forceinline__ f32x4 pack4(const f32x4& x) { return x; }
  static __device__ __forceinline__ f32x4 mma(const V8& a, const V8& b, f32x4 acc) { return mma32(a, b, acc); }
};


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

// 16 bytes read once (STREAM: a non-temporal load, so that data nobody reads
// again does not displace what the caches still hold for other waves, such as
// chunk records written a few scan steps earlier).
template <bool STREAM>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (STREAM)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// ---- hand-over of chunk records between two kernels that run at once -------
// The producer stores the record with device-scope buffer stores (the sc1
// cache-policy bit: written through to memory, so a load from another
// compute unit or XCD sees them once the store has completed) and, once every
// wave's stores have completed, adds 1 to a counter with a device-scope
// atomic.  The consumer waits until the counter reaches the number of records
// and then acquires at device scope (invalidating its caches once), after
// which plain loads see the records.  No cache-wide write-back per record.
constexpr int kDeviceScope = 16;            // buffer-op cache policy: sc1
constexpr uint32_t kPoison = 0x7FC07FC0u;  // a NaN as fp32 and as both bf16 halves
constexpr int kCountSpinLimit = 1 << 20;   // polls (about a second) before giving up

struct RecSink {
  __amdgpu_buffer_rsrc_t rsrc;  // the record (uniform)
  const char* base;
  __device__ __forceinline__ int off(const void* p) const { return (int)(static_cast<const char*>(p) - base); }
  __device__ __forceinline__ void st16(const void* p, u32x4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, off(p), 0, kDeviceScope);
  }
  __device__ __forceinline__ void st4(const void* p, float v) const {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc, off(p), 0, kDeviceScope);
  }
};
__device__ __forceinline__ RecSink rec_sink(char* rec, int bytes) {
  return RecSink{__builtin_amdgcn_make_buffer_rsrc(rec, (short)0, bytes, 0x00020000), rec};
}

// Producer side: after every wave of the workgroup has issued its record
// stores, wait for them (vmcnt(0) in each wave), then count the record.
__device__ __forceinline__ void count_record(uint32_t* done) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Consumer side (one wave per workgroup: every poll is a load of the same
// word, so few pollers, ≈0.2 µs plus a load's latency apart): wait until *done >= target, then
// acquire; the caller's workgroup barrier orders the other waves' loads after
// it.  Returns false when the bounded wait gave up (the caller then poisons
// what it stages, so that a producer that never ran shows as NaN, not a hang).
__device__ __forceinline__ bool wait_records(const uint32_t* done, uint32_t target) {
  uint32_t* d = const_cast<uint32_t*>(done);
  int spin = 0;
  bool ok = true;
  while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < target) {
    if (++spin > kCountSpinLimit) {
      ok = false;
      break;
    }
    __builtin_amdgcn_s_sleep(8);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return ok;
}

// Producer pacing (one thread per workgroup): wait until *progress >= target,
// unless pacing is off.  Performance only, never needed for correctness: the
// wait is bounded (about 200 µs), and the first wait that runs out turns
// pacing off for the whole launch (*off = 1), e.g. when the consumer is not
// running at the same time.
constexpr int kPaceSpinLimit = 128;
__device__ __forceinline__ void pace(const uint32_t* progress, uint32_t target, uint32_t* off) {
  uint32_t* pr = const_cast<uint32_t*>(progress);
  if (__hip_atomic_load(pr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return;
  if (__hip_atomic_load(off, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return;
  for (int spin = 0; __hip_atomic_load(pr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++spin) {
    if (spin >= kPaceSpinLimit) {
      __hip_atomic_store(off, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(32);
  }
}

// OR a status bit into a device-wide status word (a device-scope atomic).
__device__ __forceinline__ void raise_status(uint32_t* status, uint32_t bit) {
  if (status != nullptr) __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace kda
