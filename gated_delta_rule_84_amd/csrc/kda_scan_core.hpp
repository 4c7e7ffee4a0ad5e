// State-scan pieces shared by the scan kernel (records from HBM) and the
// fused kernel (records produced in LDS): the MFMA chain of the compute waves
// over an LDS image of the chunk record, and the gate epilogue that turns the
// chunk's fp32 output tile into o / y.
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3).  Section 2.1: per chunk with entry
// state S and the UT pair of the intra-chunk steps,
//     U'     = T Diag(beta) (V - (K . Gamma) S)      (= U - W S)
//     O      = (Q . Gamma) S + Tril(A_qk) U'
//     S_next = Diag(Gamma_last) S + (K . Gamma_last / Gamma)^T U'
// Section 2.3: y = Sigmoid(gate) . RMSNorm(o) over the d_v channels of a head.
// Rounding plan (bf16 inputs): every product takes fp16 operands -- the
// record entries, the state (held as S * 2^-4, see RecOps), the residual
// V - (K . Gamma) S and U' -- with fp32 accumulation; V enters the residual
// through an exact bf16 selection product; S stays fp32.  The fp32 path uses
// fp32 MFMA.
#pragma once

#include "kda_common.hpp"
#include "kda_params.hpp"

#include <type_traits>

namespace kda {

// Operand types of the scan's products: Opnd for the record entries and the
// operands formed from accumulators (fp16 or fp32), In8 for the V slab (the
// input type).
template <typename T>
struct ScanOps;

template <>
struct ScanOps<uint16_t> {
  using RO = RecOps<uint16_t>;
  using Opnd = f16x8;
  using In8 = bf16x8;
  static __device__ __forceinline__ Opnd ld(const char* p) { return *reinterpret_cast<const f16x8*>(p); }
  static __device__ __forceinline__ In8 ld_in(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }
  static __device__ __forceinline__ Opnd from_acc(const f32x4& a, const f32x4& b) { return RO::plain_acc(a, b); }
  static __device__ __forceinline__ f32x4 mma(const Opnd& a, const Opnd& b, f32x4 acc) { return mma32(a, b, acc); }
  static __device__ __forceinline__ f32x4 mma_in(const In8& a, const In8& b, f32x4 acc) { return mma32(a, b, acc); }
  static __device__ __forceinline__ float in_f32(uint16_t x) { return bf16_to_f32(x); }
};

template <>
struct ScanOps<float> {
  using Opnd = f32x8;
  using In8 = f32x8;
  static __device__ __forceinline__ Opnd ld(const char* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 16);
    return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
  static __device__ __forceinline__ In8 ld_in(const char* p) { return ld(p); }
  static __device__ __forceinline__ Opnd from_acc(const f32x4& a, const f32x4& b) { return acc_pair_to_f32(a, b); }
  static __device__ __forceinline__ f32x4 mma(const Opnd& a, const Opnd& b, f32x4 acc) { return mma32(a, b, acc); }
  static __device__ __forceinline__ f32x4 mma_in(const In8& a, const In8& b, f32x4 acc) { return mma32(a, b, acc); }
  static __device__ __forceinline__ float in_f32(float x) { return x; }
};

// 0/1 selection operand for the V product: K-slot j of lane group g is column
// 8 g + j of the wave's 32 columns; output column n of tile nt is column
// 16 nt + n.
template <typename V8>
__device__ __forceinline__ V8 v_select(int n, int g, int nt) {
  V8 s;
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = (8 * g + j == 16 * nt + n) ? 1.0f : 0.0f;
  return s;
}

// Compute waves of a specialised workgroup: wave `wave` (0 .. D / 32 - 1)
// owns the L::NCT 16-column tiles of value columns cb + 16 NCT wave + 0 ..
// 16 NCT - 1 (32 columns, or 16 when a head's columns are split between two
// workgroups, each with column base cb) and keeps that d_k-row slice of the
// fp32 state in accumulators for the whole sequence (scaled by
// RecOps<T>::kStateScale).  The LDS slabs (V, output tile) hold the
// workgroup's own columns.  Per chunk step, with the layout L of the LDS image:
//   first half  -- reads part A of the record (qg, kg) and the V slab;
//   barrier M   -- part A consumed, part B (kdt, tb, aq, Gamma_last) staged;
//   second half -- reads part B, writes the chunk's output tile;
//   barrier E   -- part B consumed, tile and the next part A staged.
// One barrier before the first step (part A of chunk 0 staged).  Writes the
// final state, and the prefix-cache snapshots when asked for.
template <typename T, int D, typename L>
__device__ __forceinline__ void scan_compute_waves(const ScanParams& p, char* lds, int wave, int lane, int b, int h,
                                                   int cb = 0) {
  using Ops = ScanOps<T>;
  using Opnd = typename Ops::Opnd;
  using In8 = typename Ops::In8;
  constexpr float kScale = RecOps<T>::kStateScale, kUnscale = 1.0f / RecOps<T>::kStateScale;
  constexpr int MT = D / 16;
  constexpr int KS = D / 32;
  constexpr int NCT = L::NCT;  // 16-column tiles per compute wave
  const int n = lane & 15, g4 = lane >> 4;
  const int64_t bh = (int64_t)b * p.H + h;
  const int lc0 = 16 * NCT * wave + n;  // column of tile nt in the workgroup's slabs: lc0 + 16 nt
  const int col0 = cb + lc0;            // and in the head's state
  // V enters through a 32-wide K-step over the slab columns that hold this
  // wave's tiles: window w32, tile nt at selection position vpos + nt
  const int w32 = (16 * NCT * wave) / 32 * 32, vpos = (NCT * wave) & 1;
  f32x4 S[MT][NCT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) S[mt][nt] = zero4();
  if (p.S_in != nullptr) {
    const float* s0 = p.S_in + bh * D * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mt][nt][i] = s0[(16 * mt + 4 * g4 + i) * D + col0 + 16 * nt] * kScale;
  }
  In8 vsel[NCT];
#pragma unroll
  for (int nt = 0; nt < NCT; ++nt) vsel[nt] = v_select<In8>(n, g4, vpos + nt);
  const char* qg = lds + L::QG;
  const char* kg = lds + L::KG;
  const char* kdt = lds + L::KDT;
  const char* tb = lds + L::TB;
  const char* aq = lds + L::AQ;
  const float* gam = reinterpret_cast<const float*>(lds + L::GAM);
  __syncthreads();  // part A of chunk 0 staged

  f32x4 O[4][NCT];  // outputs of the chunk
  auto write_tile = [&](int c) {  // into the tile buffer of chunk c (L::NOT buffers)
    float* otile = reinterpret_cast<float*>(lds + L::OT) + (c % L::NOT) * (64 * L::PO);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) otile[(16 * mt + 4 * g4 + i) * L::PO + lc0 + 16 * nt] = O[mt][nt][i];
  };
  for (int c = 0; c < p.nc; ++c) {
    // Every product step below issues the LDS reads of the next step's
    // operands before its own MFMAs (scheduling fences keep that order), so
    // the LDS latency overlaps the previous products.

    // R = V - (K . Gamma) S (the record holds kg negated; V enters through a
    // 0/1 selection product, rows past the end are zero) and O = (Q . Gamma) S.
    // The steps run K-step major, so only one K-step's operand of S is live.
    f32x4 R[4][NCT];
    {
      In8 av[2];
      auto ldv = [&](int mt, int bf) {
        av[bf] = Ops::ld_in(lds + L::VS + (16 * mt + n) * L::PV + (w32 + 8 * g4) * L::ES);
      };
      ldv(0, 0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int bf = mt & 1;
        if (mt + 1 < 4) ldv(mt + 1, bf ^ 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt) {
          R[mt][nt] = Ops::mma_in(av[bf], vsel[nt], zero4());
          O[mt][nt] = zero4();
        }
      }
      constexpr int G1 = 4 * KS;  // steps (kk, mt)
      Opnd ak[2], aqv[2];
      auto ld1 = [&](int g, int bf) {
        const int kk = g / 4, mt = g % 4;
        const int off = (16 * mt + n) * L::PQ + (32 * kk + 8 * g4) * L::RS;
        ak[bf] = Ops::ld(kg + off);
        aqv[bf] = Ops::ld(qg + off);
      };
      ld1(0, 0);
      Opnd Sp[NCT];
#pragma unroll
      for (int g = 0; g < G1; ++g) {
        const int bf = g & 1, kk = g / 4, mt = g % 4;
        if (g + 1 < G1) ld1(g + 1, bf ^ 1);
        if (mt == 0)
#pragma unroll
          for (int nt = 0; nt < NCT; ++nt) Sp[nt] = Ops::from_acc(S[2 * kk][nt], S[2 * kk + 1][nt]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt) {
          R[mt][nt] = Ops::mma(ak[bf], Sp[nt], R[mt][nt]);
          O[mt][nt] = Ops::mma(aqv[bf], Sp[nt], O[mt][nt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    Opnd Rp[2][NCT];
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) {
      Rp[0][nt] = Ops::from_acc(R[0][nt], R[1][nt]);
      Rp[1][nt] = Ops::from_acc(R[2][nt], R[3][nt]);
    }
    __syncthreads();  // part A of chunk c consumed; part B of chunk c staged; tile c - 1 done

    // lower-triangular (token tile, K-step) blocks of T Diag(beta) and Tril(A_qk)
    constexpr int NB = 6;
    constexpr int BMT[NB] = {0, 1, 2, 2, 3, 3}, BKK[NB] = {0, 0, 0, 1, 0, 1};
    Opnd at[2], ah[2], k0[2], k1[2];
    f32x4 gm[2];
    auto ld_t = [&](int i, int bf) { at[bf] = Ops::ld(tb + (16 * BMT[i] + n) * L::PK + (32 * BKK[i] + 8 * g4) * L::RS); };
    auto ld_a = [&](int i, int bf) { ah[bf] = Ops::ld(aq + (16 * BMT[i] + n) * L::PK + (32 * BKK[i] + 8 * g4) * L::RS); };
    auto ld_s = [&](int mt, int bf) {
      const int off = (16 * mt + n) * L::PK + 8 * g4 * L::RS;
      k0[bf] = Ops::ld(kdt + off);
      k1[bf] = Ops::ld(kdt + off + 32 * L::RS);
      gm[bf] = *reinterpret_cast<const f32x4*>(gam + 16 * mt + 4 * g4);
    };

    // U' = (T Diag(beta)) R
    Opnd Up[2][NCT];
    {
      f32x4 U[4][NCT];
      ld_t(0, 0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int bf = i & 1, mt = BMT[i], kk = BKK[i];
        if (i + 1 < NB)
          ld_t(i + 1, bf ^ 1);
        else
          ld_a(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt) U[mt][nt] = Ops::mma(at[bf], Rp[kk][nt], kk == 0 ? zero4() : U[mt][nt]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt) {
        Up[0][nt] = Ops::from_acc(U[0][nt], U[1][nt]);
        Up[1][nt] = Ops::from_acc(U[2][nt], U[3][nt]);
      }
    }

    // O += Tril(A_qk) U'
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int bf = i & 1, mt = BMT[i], kk = BKK[i];
      if (i + 1 < NB)
        ld_a(i + 1, bf ^ 1);
      else
        ld_s(0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt) O[mt][nt] = Ops::mma(ah[bf], Up[kk][nt], O[mt][nt]);
    }

    // S <- Diag(Gamma_last) S + Kd^T U'
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int bf = mt & 1;
      if (mt + 1 < MT) ld_s(mt + 1, bf ^ 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mt][nt][i] *= gm[bf][i];
        S[mt][nt] = Ops::mma(k0[bf], Up[0][nt], S[mt][nt]);
        S[mt][nt] = Ops::mma(k1[bf], Up[1][nt], S[mt][nt]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    write_tile(c);    // the helpers are done with this buffer's previous tile (barrier above)
    {
      // prefix-cache snapshot of the state after this chunk
      const int j = snapshot_index(p, p.t0 / kChunk + c);
      if (j >= 0) {
        // the lane's addresses are formed here from an opaque copy of the lane
        // id, so that they are not computed ahead and held across the loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        float* sn = p.snaps + (((int64_t)b * p.n_snap + j) * p.H + h) * D * D + 4 * (ln >> 4) * D + cb +
                    16 * NCT * wave + (ln & 15);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sn[(16 * mt + i) * D + 16 * nt] = S[mt][nt][i] * kUnscale;
      }
    }
    __syncthreads();  // part B of chunk c consumed; tile c and part A of chunk c + 1 staged
  }

  if (p.S_out == nullptr) return;
  float* so = p.S_out + bh * D * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[(16 * mt + 4 * g4 + i) * D + col0 + 16 * nt] = S[mt][nt][i] * kUnscale;
}

// Gate epilogue over the output tile of one chunk (section 2.3): NH threads,
// TPR per token row, each with EC consecutive columns of the DV columns the
// workgroup owns (DV = D, or D / 2 when a head's columns are split between
// two workgroups; cb is the first of them); the row's RMS comes from a
// shuffle reduction over its TPR threads (and, split, the other workgroup's
// half).  o is stored when asked for; y = Sigmoid(gate) . o / rms(o) . w
// when the gate is given.  LIGHT: two passes over the tile (sum of squares,
// then y in groups of 8 columns) and the RMSNorm weight read when used, for
// callers short of registers; otherwise one pass with the row segment and
// the weights in registers.  Every form sums the squares in the same order --
// sequential sums over 16-column blocks, added block by block, then the
// shuffle tree over the threads of the row -- so the split halves, the
// one-pass and the two-pass forms all round identically.
template <typename T, int D, bool OUT_F32, int NH, bool LIGHT, int DV = D>
struct GateEpilogue {
  using OutT = typename std::conditional<OUT_F32, float, uint16_t>::type;
  static constexpr int ES = sizeof(T);
  static constexpr int TPR = NH / 64;      // threads per output row
  static constexpr int EC = DV / TPR;      // columns per thread
  static constexpr int NG = EC * ES / 16;  // 16-byte vectors of gate logits per thread
  static constexpr int PER = 16 / ES;      // gate logits per 16-byte vector
  static_assert(EC % 16 == 0, "blocks of 16 columns");
  int er, ec;                              // row and first column (within the DV) of this thread
  int cb;                                  // first column of the workgroup's DV
  float wv[LIGHT ? 1 : EC];                // RMSNorm weight of those columns (one-pass form)

  __device__ __forceinline__ void init(const ScanParams& p, int h, int hid, int col_base = 0) {
    er = hid / TPR;
    ec = (hid % TPR) * EC;
    cb = col_base;
    if constexpr (!LIGHT) {
#pragma unroll
      for (int j = 0; j < EC; ++j) wv[j] = (p.rms_w != nullptr) ? p.rms_w[h * D + cb + ec + j] : 1.0f;
    }
  }

  // sum of squares of a 16-column block, sequentially
  static __device__ __forceinline__ float sumsq16(const float* x) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s = __builtin_fmaf(x[j], x[j], s);
    return s;
  }
  // over the threads of a row
  static __device__ __forceinline__ float row_reduce(float ss) {
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m);
    return ss;
  }

  // 8 values to 8 output elements (16 or 32 bytes)
  static __device__ __forceinline__ void store8(OutT* dst, const float* x) {
    if constexpr (OUT_F32) {
      reinterpret_cast<float4*>(dst)[0] = make_float4(x[0], x[1], x[2], x[3]);
      reinterpret_cast<float4*>(dst)[1] = make_float4(x[4], x[5], x[6], x[7]);
    } else {
      u32x4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = pack2_bf16(x[2 * k], x[2 * k + 1]);
      *reinterpret_cast<u32x4*>(dst) = w;
    }
  }

  static __device__ __forceinline__ float logit(const u32x4& graw, int k) {
    if constexpr (ES == 2)
      return __uint_as_float((graw[k >> 1] >> (16 * (k & 1))) << 16);
    else
      return __uint_as_float(graw[k]);
  }

  // Gate logits of this thread's row segment of the chunk at token tok0 from
  // HBM (rows past the end re-read the last row; they are never stored).
  __device__ __forceinline__ void load_gate(const ScanParams& p, int64_t head_base, int tok0, u32x4 (&g)[NG]) const {
    const int64_t tok_stride = token_stride(p.head_first, p.H, D);
    const int row = min(er, p.T - tok0 - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const T*>(p.gate) + head_base +
                                                      (int64_t)(tok0 + row) * tok_stride + cb + ec);
#pragma unroll
    for (int q = 0; q < NG; ++q) g[q] = src[q];
  }

  // this thread's 16-column block q16 of its row of the tile
  __device__ __forceinline__ void read16(const float* trow, int q16, float (&x)[16]) const {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(trow + 16 * q16 + 4 * k);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * k + j] = t[j];
    }
  }

  // y of this thread's row segment from the row's full sum of squares
  template <int PO, typename GetG>
  __device__ __forceinline__ void emit_y(const ScanParams& p, int h, int64_t orow, const float* trow, GetG getg,
                                         float ss) const {
    const float rinv = hw_rsqrt(ss / D + p.rms_eps);
#pragma unroll
    for (int q = 0; q < EC / 8; ++q) {
      float yv[8];
      const f32x4 t0 = *reinterpret_cast<const f32x4*>(trow + 8 * q);
      const f32x4 t1 = *reinterpret_cast<const f32x4*>(trow + 8 * q + 4);
      f32x4 w0 = {1.f, 1.f, 1.f, 1.f}, w1 = w0;
      if constexpr (LIGHT) {
        if (p.rms_w != nullptr) {
          w0 = *reinterpret_cast<const f32x4*>(p.rms_w + h * D + cb + ec + 8 * q);
          w1 = *reinterpret_cast<const f32x4*>(p.rms_w + h * D + cb + ec + 8 * q + 4);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          w0[j] = wv[8 * q + j];
          w1[j] = wv[8 * q + 4 + j];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = 8 * q + j;  // column within the segment
        const float ov = j < 4 ? t0[j] : t1[j - 4];
        const float w = j < 4 ? w0[j] : w1[j - 4];
        yv[j] = sigmoid_fast(logit(getg(e / PER), e % PER)) * ov * (rinv * w);
      }
      store8(static_cast<OutT*>(p.y) + orow + 8 * q, yv);
    }
  }

  // o / y of the chunk at token tok0 of head h from the tile (row pitch PO
  // floats); getg(q) returns the q-th 16-byte vector of this thread's gate
  // logits.  Only the last chunk can have rows past the end (CHECK_ROWS).
  template <bool CHECK_ROWS, int PO, typename GetG>
  __device__ __forceinline__ void run(const ScanParams& p, int h, int64_t head_base, int tok0, const float* otile,
                                      GetG getg) const {
    static_assert(DV == D, "a split row needs half_ss / emit_y");
    if (CHECK_ROWS && er >= p.T - tok0) return;
    const int64_t tok_stride = token_stride(p.head_first, p.H, D);
    const int64_t orow = head_base + (tok0 + er) * tok_stride + cb + ec;
    const float* trow = otile + er * PO + ec;
    float ss = 0.f;
#pragma unroll
    for (int q16 = 0; q16 < EC / 16; ++q16) {
      float x[16];
      read16(trow, q16, x);
      const float s16 = sumsq16(x);
      ss = q16 == 0 ? s16 : ss + s16;
      if (p.o != nullptr)
#pragma unroll
        for (int k = 0; k < 2; ++k) store8(static_cast<OutT*>(p.o) + orow + 16 * q16 + 8 * k, x + 8 * k);
    }
    if (p.y == nullptr) return;
    emit_y<PO>(p, h, orow, trow, getg, row_reduce(ss));
  }

  // Split row, first half: o of this thread's segment (when asked for) and
  // the sum of squares over the workgroup's DV columns of the row.
  template <bool CHECK_ROWS, int PO>
  __device__ __forceinline__ float half_ss(const ScanParams& p, int64_t head_base, int tok0, const float* otile) const {
    if (CHECK_ROWS && er >= p.T - tok0) return 0.f;
    const int64_t tok_stride = token_stride(p.head_first, p.H, D);
    const int64_t orow = head_base + (tok0 + er) * tok_stride + cb + ec;
    const float* trow = otile + er * PO + ec;
    float ss = 0.f;
#pragma unroll
    for (int q16 = 0; q16 < EC / 16; ++q16) {
      float x[16];
      read16(trow, q16, x);
      const float s16 = sumsq16(x);
      ss = q16 == 0 ? s16 : ss + s16;
      if (p.o != nullptr)
#pragma unroll
        for (int k = 0; k < 2; ++k) store8(static_cast<OutT*>(p.o) + orow + 16 * q16 + 8 * k, x + 8 * k);
    }
    return row_reduce(ss);
  }

  // Split row, second half: y from the tile and the row's full sum of squares.
  template <bool CHECK_ROWS, int PO, typename GetG>
  __device__ __forceinline__ void split_y(const ScanParams& p, int h, int64_t head_base, int tok0, const float* otile,
                                          GetG getg, float ss) const {
    if (CHECK_ROWS && er >= p.T - tok0) return;
    const int64_t tok_stride = token_stride(p.head_first, p.H, D);
    emit_y<PO>(p, h, head_base + (tok0 + er) * tok_stride + cb + ec, otile + er * PO + ec, getg, ss);
  }
};

}  // namespace kda
