// Inter-chunk state scan.  A workgroup of 4 waves owns 64 value columns of
// one head (16 per wave); each wave keeps its d_k x 16 slice of the fp32 state
// S in MFMA accumulators for the whole sequence and walks the chunks in order.
// The columns of S evolve independently, so waves never exchange state.  The
// chunk record written by the intra-chunk kernel, and the workgroup's 64x64
// slab of V, are copied into LDS by the whole workgroup: the loads for chunk
// c + 1 are in flight in registers while chunk c is computed from LDS, and
// are committed to LDS after it.
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
  static __device__ __forceinline__ V8 ld(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }
  static __device__ __forceinline__ V8 from_acc(const f32x4& a, const f32x4& b) { return acc_pair_to_bf16(a, b); }
  static __device__ __forceinline__ Prec prec_from_acc(const f32x4& a, const f32x4& b) {
    Prec r;
    acc_pair_split(a, b, r.hi, r.lo);
    return r;
  }
  static __device__ __forceinline__ V8 prec_main(const Prec& p) { return p.hi; }
  static __device__ __forceinline__ f32x4 mma_prec(const char* ah, const char* al, const Prec& b, f32x4 acc) {
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
  static __device__ __forceinline__ V8 ld(const char* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 16);
    return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
  static __device__ __forceinline__ V8 from_acc(const f32x4& a, const f32x4& b) { return acc_pair_to_f32(a, b); }
  static __device__ __forceinline__ Prec prec_from_acc(const f32x4& a, const f32x4& b) {
    return Prec{acc_pair_to_f32(a, b)};
  }
  static __device__ __forceinline__ V8 prec_main(const Prec& p) { return p.v; }
  static __device__ __forceinline__ f32x4 mma_prec(const char* ah, const char*, const Prec& b, f32x4 acc) {
    return mma32(ld(ah), b.v, acc);
  }
  static __device__ __forceinline__ f32x4 mma_split_b(const V8& a, const Prec& b, f32x4 acc) {
    return mma32(a, b.v, acc);
  }
  static __device__ __forceinline__ float in_f32(float x) { return x; }
};

// LDS image of one chunk record: the record's arrays with each row padded by
// 16 bytes so that the 16 rows read by one MFMA operand load hit distinct banks.
template <typename T, int D>
struct ScanLds {
  static constexpr int ES = sizeof(T);
  static constexpr int PQ = D * ES + 16;    // row pitch of qg / kg
  static constexpr int PK = 64 * ES + 16;   // row pitch of kdt / tb / aqh / aql
  static constexpr int QG = 0;
  static constexpr int KG = QG + 64 * PQ;
  static constexpr int KDT = KG + 64 * PQ;
  static constexpr int TB = KDT + D * PK;
  static constexpr int AQH = TB + 64 * PK;
  static constexpr int AQL = AQH + 64 * PK;
  static constexpr int GAM = AQL + (ES == 2 ? 64 * PK : 0);
  static constexpr int PV = 64 * ES + 16;   // row pitch of the V slab (64 columns)
  static constexpr int VS = GAM + 4 * D;
  static constexpr int BYTES = VS + 64 * PV;
  // the record, in 16-byte units, then the V slab (64 tokens x 64 columns)
  static constexpr RecLayout RL = rec_layout(ES, D);
  static constexpr int REC_UNITS = (RL.gam + 4 * D) / 16;
  static constexpr int V_UNITS = 64 * 64 * ES / 16;
  static constexpr int PER_THREAD = (REC_UNITS + V_UNITS + 255) / 256;
};

// Record byte offset of 16-byte unit u -> byte offset in the padded LDS image.
template <typename T, int D>
__device__ __forceinline__ int lds_offset_of_unit(int u) {
  using L = ScanLds<T, D>;
  constexpr RecLayout RL = L::RL;
  constexpr int RQ = D * L::ES;   // bytes per row of qg / kg
  constexpr int RK = 64 * L::ES;  // bytes per row of the 64-wide arrays
  const int b = u * 16;
  if (b < RL.kg) return L::QG + (b / RQ) * L::PQ + b % RQ;
  if (b < RL.kdt) { const int o = b - RL.kg; return L::KG + (o / RQ) * L::PQ + o % RQ; }
  if (b < RL.tb) { const int o = b - RL.kdt; return L::KDT + (o / RK) * L::PK + o % RK; }
  if (b < RL.aqh) { const int o = b - RL.tb; return L::TB + (o / RK) * L::PK + o % RK; }
  if (b < RL.aql) { const int o = b - RL.aqh; return L::AQH + (o / RK) * L::PK + o % RK; }
  if (b < RL.gam) { const int o = b - RL.aql; return L::AQL + (o / RK) * L::PK + o % RK; }
  return L::GAM + (b - RL.gam);
}

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void kda_scan_kernel(const ScanParams p) {
  using Ops = ScanOps<T>;
  using V8 = typename Ops::V8;
  using L = ScanLds<T, D>;
  constexpr int MT = D / 16;  // 16-row tiles of the state (key channels)
  constexpr int KS = D / 32;  // K-steps over key channels
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int col = 64 * blockIdx.x + 16 * wave + n;
  const int64_t bh = (int64_t)b * p.H + h;
  const bool col_ok = col < D;  // D = 64: one workgroup per head, all columns valid

  // Per-thread 16-byte units (the same for every chunk): record units first,
  // then V-slab units (VPR units per token row of the slab's 64 columns).
  constexpr int UNITS = L::REC_UNITS + L::V_UNITS;
  constexpr int VPR = 64 * L::ES / 16;
  int lofs[L::PER_THREAD];
#pragma unroll
  for (int i = 0; i < L::PER_THREAD; ++i) {
    const int u = tid + 256 * i;
    if (u < L::REC_UNITS) {
      lofs[i] = lds_offset_of_unit<T, D>(u);
    } else {
      const int vu = u - L::REC_UNITS;
      lofs[i] = L::VS + (vu / VPR) * L::PV + (vu % VPR) * 16;
    }
  }
  constexpr int FULL = UNITS / 256;  // slots that are always inside
  const bool tail_ok = tid + 256 * FULL < UNITS;
  const T* vin = static_cast<const T*>(p.v);
  u32x4 stg[L::PER_THREAD];
  auto fetch = [&](int c) {
    const char* rec = p.ws.base + (bh * p.nc + c) * p.ws.rec_bytes;
    const int tok0 = p.t0 + c * kChunk;
    const int last = min(kChunk, p.T - tok0) - 1;
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      const int u = tid + 256 * i;
      if (i < FULL || tail_ok) {
        const u32x4* src;
        if (u < L::REC_UNITS) {
          src = reinterpret_cast<const u32x4*>(rec) + u;
        } else {  // V rows past the end are clamped (zeroed when used)
          const int vu = u - L::REC_UNITS;
          const int r = min(vu / VPR, last);
          src = reinterpret_cast<const u32x4*>(vin + ((int64_t)(b * (int64_t)p.T + tok0 + r) * p.H + h) * D +
                                               64 * blockIdx.x + (vu % VPR) * (16 / L::ES));
        }
        stg[i] = *src;
      }
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i)
      if (i < FULL || tail_ok) *reinterpret_cast<u32x4*>(lds + lofs[i]) = stg[i];
  };

  // state: lane holds S[16 mt + 4 g4 + i][col]
  f32x4 S[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) S[mt] = zero4();
  if (p.S_in != nullptr && col_ok) {
    const float* s0 = p.S_in + bh * D * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] = s0[(16 * mt + 4 * g4 + i) * D + col];
  }

  fetch(0);
  commit();
  __syncthreads();

  for (int c = 0; c < p.nc; ++c) {
    const bool more = c + 1 < p.nc;
    if (more) fetch(c + 1);
    const char* base = lds;
    const char* qg = base + L::QG;
    const char* kg = base + L::KG;
    const char* kdt = base + L::KDT;
    const char* tb = base + L::TB;
    const char* aqh = base + L::AQH;
    const char* aql = base + L::AQL;
    const float* gam = reinterpret_cast<const float*>(base + L::GAM);
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
        const int off = (16 * mt + n) * L::PQ + (32 * kk + 8 * g4) * L::ES;
        X[mt] = mma32(Ops::ld(kg + off), Sb[kk], X[mt]);
        O[mt] = mma32(Ops::ld(qg + off), Sb[kk], O[mt]);
      }
    }

    // R = V - X at the accumulator positions (rows past the end: V = 0)
    f32x4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * g4 + i;
        const T vraw = *reinterpret_cast<const T*>(base + L::VS + r * L::PV + (16 * wave + n) * L::ES);
        const float vv = (r < nvalid && col_ok) ? Ops::in_f32(vraw) : 0.f;
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
        U[mt] = Ops::mma_split_b(Ops::ld(tb + (16 * mt + n) * L::PK + (32 * kk + 8 * g4) * L::ES), Rp[kk], U[mt]);
    }
    typename Ops::Prec Up[2];
    Up[0] = Ops::prec_from_acc(U[0], U[1]);
    Up[1] = Ops::prec_from_acc(U[2], U[3]);

    // O += Tril(A_qk) U'
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kk = 0; kk <= (mt >> 1); ++kk) {
        const int off = (16 * mt + n) * L::PK + (32 * kk + 8 * g4) * L::ES;
        O[mt] = Ops::mma_prec(aqh + off, aql + off, Up[kk], O[mt]);
      }

    // outputs (a full chunk stores without per-row guards)
    if (p.o != nullptr && col_ok) {
      const int64_t o0 = (int64_t)b * p.o_b_stride + (int64_t)(tok0 - p.o_t0) * p.o_tok_stride + h * D + col;
      const bool full = nvalid == kChunk;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mt + 4 * g4 + i;
          if (full || r < nvalid) {
            const int64_t oi = o0 + (int64_t)r * p.o_tok_stride;
            if (p.o_f32)
              static_cast<float*>(p.o)[oi] = O[mt][i];
            else
              static_cast<uint16_t*>(p.o)[oi] = f32_to_bf16(O[mt][i]);
          }
        }
    }

    // S <- Diag(Gamma_last) S + Kd^T U'
    const V8 Ub0 = Ops::prec_main(Up[0]);
    const V8 Ub1 = Ops::prec_main(Up[1]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 gm = *reinterpret_cast<const f32x4*>(gam + 16 * mt + 4 * g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] *= gm[i];
      const int off = (16 * mt + n) * L::PK + 8 * g4 * L::ES;
      S[mt] = mma32(Ops::ld(kdt + off), Ub0, S[mt]);
      S[mt] = mma32(Ops::ld(kdt + off + 32 * L::ES), Ub1, S[mt]);
    }

    if (more) {
      __syncthreads();  // every wave is done reading chunk c from LDS
      commit();
      __syncthreads();
    }
  }

  if (col_ok) {
    float* so = p.S_out + bh * D * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[(16 * mt + 4 * g4 + i) * D + col] = S[mt][i];
  }
}

hipError_t launch_scan(const ScanParams& p, int D, int in_f32, hipStream_t s) {
  const dim3 grid((D + 63) / 64, p.H, p.B), block(256);
  if (in_f32) {
    if (D == 64) hipLaunchKernelGGL((kda_scan_kernel<float, 64>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((kda_scan_kernel<float, 128>), grid, block, 0, s, p);
  } else {
    if (D == 64) hipLaunchKernelGGL((kda_scan_kernel<uint16_t, 64>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((kda_scan_kernel<uint16_t, 128>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kda
