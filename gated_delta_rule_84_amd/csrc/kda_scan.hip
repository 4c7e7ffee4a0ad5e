// Inter-chunk state scan.  Each wave owns 16 value columns of one head's
// state S (d_k x 16, fp32, kept in MFMA accumulators for the whole sequence)
// and walks the chunks in order.  The columns of S evolve independently, so
// the waves of one head never communicate.
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3), section 2.1: per chunk with entry
// state S and the UT pair of the intra-chunk kernel,
//     U'     = T Diag(beta) (V - (K . Gamma) S)      (= U - W S)
//     O      = (Q . Gamma) S + Tril(A_qk) U'
//     S_next = Diag(Gamma_last) S + (K . Gamma_last / Gamma)^T U'
// Rounding plan (bf16 path): S, K . Gamma, Q . Gamma and U' enter bf16 MFMAs
// with fp32 accumulation; the residual V - (K . Gamma) S is split into hi/lo
// bf16 parts (two products); Tril(A_qk) U' uses hi/lo split operands on both
// sides; S itself stays fp32.  The fp32 path uses fp32 MFMA.
#include "kda_common.hpp"
#include "kda_params.hpp"

namespace kda {

template <typename T>
struct ScanOps;

template <>
struct ScanOps<uint16_t> {
  using V8 = bf16x8;
  struct Prec {  // operand of the split product
    bf16x8 hi, lo;
  };
  static __device__ __forceinline__ V8 ld(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
  static __device__ __forceinline__ V8 from_acc(const f32x4& a, const f32x4& b) { return acc_pair_to_bf16(a, b); }
  static __device__ __forceinline__ Prec prec_from_acc(const f32x4& a, const f32x4& b) {
    Prec r;
    acc_pair_split(a, b, r.hi, r.lo);
    return r;
  }
  static __device__ __forceinline__ V8 prec_main(const Prec& p) { return p.hi; }
  static __device__ __forceinline__ f32x4 mma_prec(const uint16_t* ah, const uint16_t* al, const Prec& b,
                                                   f32x4 acc) {
    return mma32_x3(ld(ah), ld(al), b.hi, b.lo, acc);
  }
  // a (bf16) times a split operand: a * hi + a * lo
  static __device__ __forceinline__ f32x4 mma_split_b(const V8& a, const Prec& b, f32x4 acc) {
    acc = mma32(a, b.lo, acc);
    return mma32(a, b.hi, acc);
  }
  static __device__ __forceinline__ float in_f32(uint16_t x) { return bf16_to_f32(x); }
};

template <>
struct ScanOps<float> {
  using V8 = f32x8;
  struct Prec {
    f32x8 v;
  };
  static __device__ __forceinline__ V8 ld(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
  static __device__ __forceinline__ V8 from_acc(const f32x4& a, const f32x4& b) { return acc_pair_to_f32(a, b); }
  static __device__ __forceinline__ Prec prec_from_acc(const f32x4& a, const f32x4& b) {
    return Prec{acc_pair_to_f32(a, b)};
  }
  static __device__ __forceinline__ V8 prec_main(const Prec& p) { return p.v; }
  static __device__ __forceinline__ f32x4 mma_prec(const float* ah, const float*, const Prec& b, f32x4 acc) {
    return mma32(ld(ah), b.v, acc);
  }
  static __device__ __forceinline__ f32x4 mma_split_b(const V8& a, const Prec& b, f32x4 acc) {
    return mma32(a, b.v, acc);
  }
  static __device__ __forceinline__ float in_f32(float x) { return x; }
};

template <typename T, int D, int WPB>
__global__ __launch_bounds__(64 * WPB) void kda_scan_kernel(const ScanParams p) {
  using Ops = ScanOps<T>;
  using V8 = typename Ops::V8;
  constexpr int MT = D / 16;  // 16-row tiles of the state (key channels)
  constexpr int KS = D / 32;  // K-steps over key channels

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int v0 = 16 * (blockIdx.x * WPB + wave);
  const int col = v0 + n;
  const int64_t bh = (int64_t)b * p.H + h;

  // state: lane holds S[16 mt + 4 g4 + i][col]
  f32x4 S[MT];
  if (p.S_in != nullptr) {
    const float* s0 = p.S_in + bh * D * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] = s0[(16 * mt + 4 * g4 + i) * D + col];
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) S[mt] = zero4();
  }

  const T* vin = static_cast<const T*>(p.v);
  for (int c = 0; c < p.nc; ++c) {
    const int64_t rec = bh * p.nc + c;
    const T* qg = static_cast<const T*>(p.ws.qg) + rec * p.ws.rec_elems_qk;
    const T* kg = static_cast<const T*>(p.ws.kg) + rec * p.ws.rec_elems_qk;
    const T* kdt = static_cast<const T*>(p.ws.kdt) + rec * p.ws.rec_elems_qk;
    const T* tb = static_cast<const T*>(p.ws.tb) + rec * p.ws.rec_elems_t;
    const T* aqh = static_cast<const T*>(p.ws.aqh) + rec * p.ws.rec_elems_t;
    const T* aql = (p.ws.aql != nullptr) ? static_cast<const T*>(p.ws.aql) + rec * p.ws.rec_elems_t : aqh;
    const float* gam = p.ws.gam + rec * D;
    const int tok0 = p.t0 + c * kChunk;
    const int nvalid = min(kChunk, p.T - tok0);

    // B operands from the state, K-slots in slot order
    V8 Sb[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) Sb[kk] = Ops::from_acc(S[2 * kk], S[2 * kk + 1]);

    // X = (K . Gamma) S and O = (Q . Gamma) S; tokens on M
    f32x4 X[4], O[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      X[mt] = zero4();
      O[mt] = zero4();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int off = (16 * mt + n) * D + 32 * kk + 8 * g4;
        X[mt] = mma32(Ops::ld(kg + off), Sb[kk], X[mt]);
        O[mt] = mma32(Ops::ld(qg + off), Sb[kk], O[mt]);
      }
    }

    // R = V - X at the accumulator positions (rows past the end read as 0)
    f32x4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * g4 + i;
        float vv = 0.f;
        if (r < nvalid) vv = Ops::in_f32(vin[((int64_t)(b * (int64_t)p.T + tok0 + r) * p.H + h) * D + col]);
        R[mt][i] = vv - X[mt][i];
      }
    typename Ops::Prec Rp[2];
    Rp[0] = Ops::prec_from_acc(R[0], R[1]);
    Rp[1] = Ops::prec_from_acc(R[2], R[3]);

    // U' = (T Diag(beta)) R   (block lower triangular: tile mt needs steps <= mt/2)
    f32x4 U[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      U[mt] = zero4();
#pragma unroll
      for (int kk = 0; kk <= (mt >> 1); ++kk)
        U[mt] = Ops::mma_split_b(Ops::ld(tb + (16 * mt + n) * kChunk + 32 * kk + 8 * g4), Rp[kk], U[mt]);
    }
    typename Ops::Prec Up[2];
    Up[0] = Ops::prec_from_acc(U[0], U[1]);
    Up[1] = Ops::prec_from_acc(U[2], U[3]);

    // O += Tril(A_qk) U'
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kk = 0; kk <= (mt >> 1); ++kk) {
        const int off = (16 * mt + n) * kChunk + 32 * kk + 8 * g4;
        O[mt] = Ops::mma_prec(aqh + off, aql + off, Up[kk], O[mt]);
      }

    // outputs
    if (p.o != nullptr)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * g4 + i;
        if (r < nvalid) {
          const int64_t oi = (int64_t)b * p.o_b_stride + (int64_t)(tok0 + r - p.o_t0) * p.o_tok_stride + h * D + col;
          if (p.o_f32)
            static_cast<float*>(p.o)[oi] = O[mt][i];
          else
            static_cast<uint16_t*>(p.o)[oi] = f32_to_bf16(O[mt][i]);
        }
      }

    // S <- Diag(Gamma_last) S + Kd^T U'
    const V8 Ub0 = Ops::prec_main(Up[0]);
    const V8 Ub1 = Ops::prec_main(Up[1]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] *= gam[16 * mt + 4 * g4 + i];
      const int off = (16 * mt + n) * kChunk + 8 * g4;
      S[mt] = mma32(Ops::ld(kdt + off), Ub0, S[mt]);
      S[mt] = mma32(Ops::ld(kdt + off + 32), Ub1, S[mt]);
    }
  }

  float* so = p.S_out + bh * D * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) so[(16 * mt + 4 * g4 + i) * D + col] = S[mt][i];
}

hipError_t launch_scan(const ScanParams& p, int D, int in_f32, hipStream_t s) {
  constexpr int WPB = 2;
  const dim3 grid(D / (16 * WPB), p.H, p.B), block(64 * WPB);
  if (in_f32) {
    if (D == 64) hipLaunchKernelGGL((kda_scan_kernel<float, 64, WPB>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((kda_scan_kernel<float, 128, WPB>), grid, block, 0, s, p);
  } else {
    if (D == 64) hipLaunchKernelGGL((kda_scan_kernel<uint16_t, 64, WPB>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((kda_scan_kernel<uint16_t, 128, WPB>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kda
