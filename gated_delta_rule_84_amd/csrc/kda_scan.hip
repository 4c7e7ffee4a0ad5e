// Inter-chunk state scan with the fused output gate.  One workgroup per
// (batch, head).  Each compute wave owns a set of value columns and keeps its
// d_k x columns slice of the fp32 state S in MFMA accumulators for the whole
// sequence; the columns of S evolve independently, so waves never exchange
// state.  The chunk record written by the intra-chunk kernel and the head's
// 64 x D slab of V are staged into LDS (padded rows) one chunk ahead; the
// chunk's outputs go through an LDS tile so that the RMSNorm over a row and
// the stores of o / y are done row by row with contiguous 16-byte stores.
//
// Two organisations of the workgroup:
//  * specialised (whenever the LDS image fits): D / 32 compute waves with 32
//    columns each run only the MFMA chain, while as many helper waves load
//    the next chunk's record, V and this chunk's gate logits into registers,
//    turn the previous chunk's output tile into o / y, and commit the loads to
//    LDS between two barriers;
//  * serial (fp32 at d = 128): D / 16 waves with 16 columns each do all of it
//    in turn.
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3).  Section 2.1: per chunk with entry
// state S and the UT pair of the intra-chunk kernel,
//     U'     = T Diag(beta) (V - (K . Gamma) S)      (= U - W S)
//     O      = (Q . Gamma) S + Tril(A_qk) U'
//     S_next = Diag(Gamma_last) S + (K . Gamma_last / Gamma)^T U'
// Section 2.3: y = Sigmoid(gate) . RMSNorm(o) over the d_v channels of a head.
// Rounding plan (bf16 inputs): fp16 record entries, state and residual
// operands with fp32 accumulation (RecOps, kda_scan_core.hpp); S stays fp32.
// The fp32 path uses fp32 MFMA.
#include "kda_scan_core.hpp"

namespace kda {

// LDS image of one chunk record (rows padded by 16 bytes so that the 16 rows
// read by one MFMA operand load hit distinct banks), the V slab and the output
// tile.
template <typename T, int D>
struct ScanLds {
  static constexpr int ES = sizeof(T);     // input element (V slab)
  static constexpr int RS = sizeof(typename RecOps<T>::Elem);  // record element
  static_assert(RS == ES, "one row pitch for the record and the V slab");
  static constexpr int NT = 4 * D;          // threads (D / 16 waves)
  static constexpr int PQ = D * ES + 16;    // row pitch of qg / kg / V slab
  static constexpr int PK = 64 * RS + 16;   // row pitch of kdt / tb / aq
  static constexpr int QG = 0;
  static constexpr int KG = QG + 64 * PQ;
  static constexpr int KDT = KG + 64 * PQ;
  static constexpr int TB = KDT + D * PK;
  static constexpr int AQ = TB + 64 * PK;
  static constexpr int GAM = AQ + 64 * PK;
  static constexpr int REC = GAM + 4 * D;   // end of the record image
  static constexpr int PO = D + 4;          // fp32 output tile [64][D + 4]
  static constexpr int LIMIT = 160 * 1024;
  // The V slab goes through LDS when it fits (else straight to registers),
  // and the output tile shares the record's space when a separate one does not.
  static constexpr bool V_LDS = REC + 64 * PQ <= LIMIT;
  static constexpr int VS = REC;
  static constexpr int AFTER_V = REC + (V_LDS ? 64 * PQ : 0);
  static constexpr bool O_ALIAS = AFTER_V + 64 * PO * 4 > LIMIT;
  static constexpr int OT = O_ALIAS ? QG : AFTER_V;
  static constexpr int BYTES = O_ALIAS ? AFTER_V : AFTER_V + 64 * PO * 4;
  static_assert(BYTES <= LIMIT, "scan LDS image too large");
  static_assert(!O_ALIAS || 64 * PO * 4 <= KDT, "aliased output tile must fit in qg / kg");
  static constexpr RecUnits RU = rec_units(RS, D);
  static constexpr int REC_UNITS = RU.units;   // 16-byte units
  static constexpr int V_UNITS = V_LDS ? 64 * D * ES / 16 : 0;
  static constexpr int UNITS = REC_UNITS + V_UNITS;
  static constexpr int PER_THREAD = (UNITS + NT - 1) / NT;
  static constexpr int FULL = UNITS / NT;  // unit slots that are always in range
  // epilogue: TPR threads per token row, 16 columns each
  static constexpr int TPR = NT / 64;
  static constexpr int GV = 16 * ES / 16;  // 16-byte vectors of gate logits per thread
};

// Record unit u (the workspace layout of rec_units) -> byte offset in the
// padded LDS image.  A 2-byte unit of Kd^T carries two 8-byte pieces: the
// offset is the first one's; the second goes 16 rows further down (KDT_SECOND
// beyond it).
template <typename L, int D>
__device__ __forceinline__ int lds_offset_of_unit(int u) {
  constexpr RecUnits RU = L::RU;
  constexpr int KS = D / 32, UPP = L::RS / 2;  // units per 8-element piece
  if (u < RU.tb) {  // qg, kg, kdt: piece (ti, kk, lane), part h of it (fp32)
    const int region = u < RU.kg ? 0 : u < RU.kdt ? 1 : 2;
    const int v = u - (region == 0 ? RU.qg : region == 1 ? RU.kg : RU.kdt);
    const int pc = v / UPP, h = v % UPP;
    const int ti = pc / (64 * KS), kk = (pc / 64) % KS, lane = pc % 64;
    const int n = lane & 15, g4 = lane >> 4;
    if (region < 2) return (region == 0 ? L::QG : L::KG) + (16 * ti + n) * L::PQ + (32 * kk + 8 * g4 + 4 * h) * L::RS;
    const int tpos = 32 * (ti >> 1) + 8 * g4 + 4 * (ti & 1);
    return L::KDT + (32 * kk + 16 * h + n) * L::PK + tpos * L::RS;
  }
  if (u < RU.aq) {  // T Diag(beta): 32 slots of rows 0..31, then 64 slots of rows 32..63
    constexpr int W32 = 32 * L::RS / 16, W64 = 64 * L::RS / 16;
    const int v = u - RU.tb;
    const int rr = v < 32 * W32 ? v / W32 : 32 + (v - 32 * W32) / W64;
    const int w = v < 32 * W32 ? v % W32 : (v - 32 * W32) % W64;
    return L::TB + rr * L::PK + 16 * w;
  }
  if (u < RU.gam) {  // Tril(A_qk): piece (group, lane), part h of it (fp32)
    const int v = u - RU.aq;
    const int pc = v / UPP, h = v % UPP;
    const int grp = pc / 64, lane = pc % 64;
    const int ti = aq_group_tile(grp), pr = aq_group_pair(grp);
    const int n = lane & 15, g4 = lane >> 4;
    return L::AQ + (16 * ti + n) * L::PK + (32 * pr + 8 * g4 + 4 * h) * L::RS;
  }
  return L::GAM + 16 * (u - RU.gam);
}

// 16 consecutive fp32 values -> 16 outputs (fp32 or bf16) at dst.
__device__ __forceinline__ void store16(void* dst, const float* x, int out_f32) {
  if (out_f32) {
    float4* d = static_cast<float4*>(dst);
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
  } else {
    u32x4 w[2];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      w[q >> 2][q & 3] = pack2_bf16(x[2 * q], x[2 * q + 1]);
    u32x4* d = static_cast<u32x4*>(dst);
    d[0] = w[0];
    d[1] = w[1];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(4 * D, 1) void kda_scan_serial_kernel(const ScanParams p) {
  using Ops = ScanOps<T>;
  using Opnd = typename Ops::Opnd;
  using L = ScanLds<T, D>;
  static_assert(sizeof(T) == 4, "one LDS place per record unit: fp32 records");
  constexpr int MT = D / 16;  // 16-row tiles of the state (key channels)
  constexpr int KS = D / 32;  // K-steps over key channels
  constexpr int NT = L::NT;
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int h = blockIdx.x, b = blockIdx.y;
  const int col = 16 * wave + n;
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t tok_stride = token_stride(p.head_first, p.H, D);  // elements between tokens of one head
  const int64_t head_base = token_base(p.head_first, b, h, p.T, p.H, D);

  // ---- per-thread copy units: record units, then V-slab units -------------
  constexpr int VPR = D * L::ES / 16;  // 16-byte units per V row
  int lofs[L::PER_THREAD];
#pragma unroll
  for (int i = 0; i < L::PER_THREAD; ++i) {
    const int u = tid + NT * i;
    if (u < L::REC_UNITS) {
      lofs[i] = lds_offset_of_unit<ScanLds<T, D>, D>(u);
    } else {
      const int vu = u - L::REC_UNITS;
      lofs[i] = L::VS + (vu / VPR) * L::PQ + (vu % VPR) * 16;
    }
  }
  const bool tail_ok = tid + NT * L::FULL < L::UNITS;
  const T* vin = static_cast<const T*>(p.v);
  u32x4 stg[L::PER_THREAD];
  // records of a producer running at the same time: wave 0 waits until all
  // are written; the barrier orders every wave's record loads after that
  __shared__ int gave_up;
  bool poison = false;
  if (p.done != nullptr) {
    if (wave == 0) {
      const bool ok = wait_records(p.done + bh, (uint32_t)p.nc);
      if (lane == 0) gave_up = ok ? 0 : 1;
      if (!ok && lane == 0) raise_status(p.status, kStatusWaitGaveUp);
    }
    __syncthreads();
    poison = gave_up != 0;
  }
  auto fetch = [&](int c) {
    const char* rec = p.ws.base + (bh * p.nc + c) * p.ws.rec_bytes;
    const int tok0 = p.t0 + c * kChunk;
    const int last = min(kChunk, p.T - tok0) - 1;
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      const int u = tid + NT * i;
      if (i < L::FULL || tail_ok) {
        if (u < L::REC_UNITS) {
          stg[i] = reinterpret_cast<const u32x4*>(rec)[u];
        } else if (vin != nullptr) {  // V rows past the end are clamped (and zeroed where used)
          const int vu = u - L::REC_UNITS;
          const int r = min(vu / VPR, last);
          stg[i] = reinterpret_cast<const u32x4*>(vin + head_base + (tok0 + r) * tok_stride)[vu % VPR];
        } else {  // no V: V = 0
          stg[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto commit = [&]() {
    if (poison)  // wave-uniform: the records never became complete
#pragma unroll
      for (int i = 0; i < L::PER_THREAD; ++i) stg[i] = u32x4{kPoison, kPoison, kPoison, kPoison};
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i)
      if (i < L::FULL || tail_ok) *reinterpret_cast<u32x4*>(lds + lofs[i]) = stg[i];
  };

  // ---- epilogue role: token row er, columns ec .. ec + 15 -----------------
  const int er = tid / L::TPR, ec = (tid % L::TPR) * 16;
  const bool gated = p.y != nullptr;
  float wv[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) wv[j] = (gated && p.rms_w != nullptr) ? p.rms_w[h * D + ec + j] : 1.0f;
  const T* gin = static_cast<const T*>(p.gate);

  // ---- state: lane holds S[16 mt + 4 g4 + i][col] ---------------------------
  f32x4 S[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) S[mt] = zero4();
  if (p.S_in != nullptr) {
    const float* s0 = p.S_in + bh * D * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] = s0[(16 * mt + 4 * g4 + i) * D + col];
  }

  fetch(0);
  commit();
  __syncthreads();

  const char* qg = lds + L::QG;
  const char* kg = lds + L::KG;
  const char* kdt = lds + L::KDT;
  const char* tb = lds + L::TB;
  const char* aq = lds + L::AQ;
  const float* gam = reinterpret_cast<const float*>(lds + L::GAM);
  float* otile = reinterpret_cast<float*>(lds + L::OT);

  for (int c = 0; c < p.nc; ++c) {
    const bool more = c + 1 < p.nc;
    const int tok0 = p.t0 + c * kChunk;
    const int nvalid = min(kChunk, p.T - tok0);

    // gate logits of this chunk for the epilogue (issued before the prefetch
    // so that waiting for them does not wait for the prefetch)
    u32x4 gvec[L::GV];
    if (gated) {
      const u32x4* src =
          reinterpret_cast<const u32x4*>(gin + head_base + (tok0 + min(er, nvalid - 1)) * tok_stride + ec);
#pragma unroll
      for (int q = 0; q < L::GV; ++q) gvec[q] = src[q];
    }
    T vreg[16];  // V at the accumulator positions when it does not go through LDS
    if constexpr (!L::V_LDS) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vreg[4 * mt + i] =
              vin ? vin[head_base + (tok0 + min(16 * mt + 4 * g4 + i, nvalid - 1)) * tok_stride + col] : T{};
    }
    if (more) fetch(c + 1);

    // B operands from the state, K-slots in slot order
    Opnd Sb[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) Sb[kk] = Ops::from_acc(S[2 * kk], S[2 * kk + 1]);

    // X = -(K . Gamma) S (the record holds kg negated) and O = (Q . Gamma) S
    f32x4 X[4], O[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      X[mt] = zero4();
      O[mt] = zero4();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int off = (16 * mt + n) * L::PQ + (32 * kk + 8 * g4) * L::RS;
        X[mt] = Ops::mma(Ops::ld(kg + off), Sb[kk], X[mt]);
        O[mt] = Ops::mma(Ops::ld(qg + off), Sb[kk], O[mt]);
      }
    }

    // R = V - X at the accumulator positions (rows past the end: V = 0)
    f32x4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * g4 + i;
        T vraw;
        if constexpr (L::V_LDS)
          vraw = *reinterpret_cast<const T*>(lds + L::VS + r * L::PQ + col * L::ES);
        else
          vraw = vreg[4 * mt + i];
        R[mt][i] = (r < nvalid ? Ops::in_f32(vraw) : 0.f) + X[mt][i];
      }
    Opnd Rp[2];
    Rp[0] = Ops::from_acc(R[0], R[1]);
    Rp[1] = Ops::from_acc(R[2], R[3]);

    // U' = (T Diag(beta)) R   (block lower triangular: tile mt needs steps <= mt/2)
    f32x4 U[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      U[mt] = zero4();
#pragma unroll
      for (int kk = 0; kk <= (mt >> 1); ++kk)
        U[mt] = Ops::mma(Ops::ld(tb + (16 * mt + n) * L::PK + (32 * kk + 8 * g4) * L::RS), Rp[kk], U[mt]);
    }
    Opnd Up[2];
    Up[0] = Ops::from_acc(U[0], U[1]);
    Up[1] = Ops::from_acc(U[2], U[3]);

    // O += Tril(A_qk) U'
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kk = 0; kk <= (mt >> 1); ++kk) {
        const int off = (16 * mt + n) * L::PK + (32 * kk + 8 * g4) * L::RS;
        O[mt] = Ops::mma(Ops::ld(aq + off), Up[kk], O[mt]);
      }

    // S <- Diag(Gamma_last) S + Kd^T U'
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 gm = *reinterpret_cast<const f32x4*>(gam + 16 * mt + 4 * g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] *= gm[i];
      const int off = (16 * mt + n) * L::PK + 8 * g4 * L::RS;
      S[mt] = Ops::mma(Ops::ld(kdt + off), Up[0], S[mt]);
      S[mt] = Ops::mma(Ops::ld(kdt + off + 32 * L::RS), Up[1], S[mt]);
    }

    // prefix-cache snapshot of the state after this chunk
    {
      const int j = snapshot_index(p, p.t0 / kChunk + c);
      if (j >= 0) {
        float* sn = p.snaps + (((int64_t)b * p.n_snap + j) * p.H + h) * D * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sn[(16 * mt + 4 * g4 + i) * D + col] = S[mt][i];
      }
    }

    // O tile to LDS (when it shares the record's space, wait until no wave
    // reads the record any more)
    if constexpr (L::O_ALIAS) __syncthreads();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) otile[(16 * mt + 4 * g4 + i) * L::PO + col] = O[mt][i];
    __syncthreads();  // O tile complete; chunk c's record and V are no longer read

    // epilogue: row er, columns ec .. ec + 15
    {
      float ov[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(otile + er * L::PO + ec + 4 * q);
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[4 * q + j] = t[j];
      }
      const bool row_ok = er < nvalid;
      const int64_t orow = head_base + (tok0 + er) * tok_stride + ec;
      if (p.o != nullptr && row_ok) {
        if (p.out_f32)
          store16(static_cast<float*>(p.o) + orow, ov, 1);
        else
          store16(static_cast<uint16_t*>(p.o) + orow, ov, 0);
      }
      if (gated) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) ss += ov[j] * ov[j];
#pragma unroll
        for (int m = 1; m < L::TPR; m <<= 1) ss += __shfl_xor(ss, m);
        const float rinv = hw_rsqrt(ss / D + p.rms_eps);
        const T* gt = reinterpret_cast<const T*>(gvec);
        float yv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) yv[j] = sigmoid_fast(Ops::in_f32(gt[j])) * ov[j] * rinv * wv[j];
        if (row_ok) {
          if (p.out_f32)
            store16(static_cast<float*>(p.y) + orow, yv, 1);
          else
            store16(static_cast<uint16_t*>(p.y) + orow, yv, 0);
        }
      }
    }

    if (more) {
      if constexpr (L::O_ALIAS) __syncthreads();  // the O tile lives in the record's space
      commit();  // nobody reads chunk c's record or V any more
      __syncthreads();
    }
  }

  float* so = p.S_out + bh * D * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) so[(16 * mt + 4 * g4 + i) * D + col] = S[mt][i];
}


// ---- specialised workgroup: compute waves + helper waves -------------------
// LDS: the padded record image (as above), the V slab of the current chunk,
// the gate-logit slab of the previous chunk, the previous chunk's fp32 output
// tile.  NCW compute waves (32 columns each) and as many helper waves.
//
// NS = 2 splits a head's value columns between two workgroups (half s owns
// columns s D / 2 .. (s + 1) D / 2 - 1; grid mapping in the kernel): every product
// of the chunk form is separable in the value columns, so each keeps half of
// the state and reads the whole record but only its half of V, the gate and
// y; its compute waves own 16 columns each, which halves their product chain.
// RMSNorm needs the whole row: each workgroup publishes the sum of squares
// of its half of every row of chunk c - 1 during step c and reads the other
// half's during step c + 1 (so the exchange's latency is hidden), then
// writes y of chunk c - 1; the output tiles and gate slabs are therefore
// double-buffered.  The sums go through a ring of four chunks per
// workgroup in the workspace as 8-byte (value, chunk + 1) words written and
// read with device-scope atomics, so a word is never seen half written and a
// stale one never matches; one workgroup can run at most two chunk steps
// ahead of the other, so four slots are never overwritten before they are
// read.  Both workgroups of a pair must be resident together: the host uses
// the split only for one-stream launches with 2 B H within the device's
// compute units, and the wait is bounded (status bit, NaN y).  The sums of
// squares are formed in the same order as the unsplit epilogue's, so results
// are bit-identical.
//
// The staging is split in two parts so that it never stalls the compute waves:
// part A (qg, kg of the record and the V slab) is read in the first half of a
// chunk step, part B (kdt, tb, aq, Gamma_last) in the second half.  Helpers
// commit part B of chunk c during the first half of step c, and part A of
// chunk c + 1 with chunk c's gate logits during the second half; each part is
// loaded into registers one step before it is committed.  The helpers turn
// chunk c - 1's output tile into o / y during the first half of step c, while
// the compute waves run the long independent product chains of chunk c.
template <typename T, int D, int NS = 1>
struct WsLds {
  static constexpr int ES = sizeof(T);
  static constexpr int DV = D / NS;            // value columns of the workgroup
  static constexpr int NCT = 2 / NS;           // 16-column tiles per compute wave
  static constexpr int NCW = D / 32;           // compute waves
  static constexpr int NHW = NCW;              // helper waves
  static constexpr int NT = 64 * (NCW + NHW);  // threads
  static constexpr int NH = 64 * NHW;          // helper threads
  static constexpr int RS = sizeof(typename RecOps<T>::Elem);  // record element
  static_assert(RS == ES, "one row pitch for the record and the slabs");
  // Row padding of the LDS image: 32 bytes make the compute waves' operand
  // reads (lane (n, g) reads 16 bytes of row n at column group g) take 4 LDS
  // cycles instead of 8; that pays only in the split workgroup (its scan
  // alone: -3.5%), while the unsplit one beside the intra kernel measured
  // 1% slower with it (LDS 149 vs 141 KB)
  static constexpr int PAD = NS == 2 ? 32 : 16;
  static constexpr int PQ = D * ES + PAD;
  static constexpr int PK = 64 * RS + PAD;
  static constexpr int QG = 0;
  static constexpr int KG = QG + 64 * PQ;
  static constexpr int KDT = KG + 64 * PQ;
  static constexpr int TB = KDT + D * PK;
  static constexpr int AQ = TB + 64 * PK;
  static constexpr int GAM = AQ + 64 * PK;
  static constexpr int REC = GAM + 4 * D;
  static constexpr int PV = DV * ES + PAD;     // row pitch of the V and gate slabs
  static constexpr int NOT = NS;               // gate slabs and output tiles (double-buffered when split)
  static constexpr int VS = REC;               // V slab   [64][PV]
  static constexpr int GS = VS + 64 * PV;      // gate slabs [NOT][64][PV]
  static constexpr int PO = DV + 4;
  static constexpr int OT = GS + NOT * 64 * PV;  // output tiles [NOT][64][PO] fp32
  static constexpr int FLAG = OT + NOT * 64 * PO * 4;  // outcome of the record waits (int)
  static constexpr int BYTES = FLAG + 16;
  static constexpr RecUnits RU = rec_units(RS, D);
  static constexpr int VPR = DV * ES / 16;     // 16-byte units per slab row
  static constexpr int SLAB_UNITS = 64 * VPR;
  static constexpr int A_REC = RU.kdt;         // record units of part A (qg, kg)
  static constexpr int A_UNITS = A_REC + SLAB_UNITS;
  static constexpr int B_UNITS = RU.units - RU.kdt;
  // part B (relative units): Kd^T (split, whole steps), then T Diag(beta),
  // Tril(A_qk) and Gamma_last (plain)
  static constexpr int KDT_STEPS = (RU.tb - RU.kdt) / NH;
  static constexpr int KDT_SECOND = 16 * PK;   // second piece of a Kd^T unit: 16 rows down
  static constexpr int PA = (A_UNITS + NH - 1) / NH;
  static constexpr int PB = (B_UNITS + NH - 1) / NH;
  static constexpr int PG = (SLAB_UNITS + NH - 1) / NH;
  static constexpr int TPR = NH / 64;          // helper threads per output row
  static constexpr int EC = DV / TPR;          // columns per helper thread
  // used when the image fits in LDS and a helper's staging registers stay modest
  static constexpr bool FITS = BYTES <= 160 * 1024 && PA + PB + PG <= 40;
};

template <typename T, int D, bool OUT_F32, int NS>
__global__ __launch_bounds__((WsLds<T, D, NS>::NT), 1) void kda_scan_ws_kernel(const ScanParams p) {
  using L = WsLds<T, D, NS>;
  static_assert(sizeof(typename RecOps<T>::Elem) == 2, "the split commits of part B assume 2-byte records");
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // NS = 2: a 1-D grid of groups of 16 workgroups, 8 heads each: workgroup
  // 16 g + 8 s + r takes half s of head (b, h) = pair 8 g + r, so that the two
  // halves of a head, which read the same chunk records, are dispatched to the
  // same XCD (workgroups go to the XCDs in turn) and share its L2.  Workgroups
  // past the last pair return at once.
  int h = blockIdx.x, b = blockIdx.y, half = 0;
  if constexpr (NS == 2) {
    const int pair = 8 * ((int)blockIdx.x / 16) + (int)blockIdx.x % 8;
    if (pair >= p.B * p.H) return;
    half = ((int)blockIdx.x / 8) & 1;
    b = pair / p.H;
    h = pair % p.H;
  }
  const int cb = half * L::DV;            // first column of the workgroup's half
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t tok_stride = token_stride(p.head_first, p.H, D);
  const int64_t head_base = token_base(p.head_first, b, h, p.T, p.H, D);

  // Records of a producer running at the same time: the first helper wave
  // waits until they are written, and a workgroup barrier orders every
  // wave's record loads after that.  The overlapped schedule waits here for
  // the whole launch; the pipelined schedule waits here for the segments of
  // chunks 0 and 1 (the prologue loads) and, in the helper loop, for each
  // later segment two chunk steps before its first record is loaded.  The
  // outcome goes through an LDS word; a wait that gave up poisons what the
  // helpers stage from then on (and no later wait is made).
  const int n_seg = p.seg_len > 0 ? num_segments(p.nc, p.seg_len) : 0;
  auto seg_start = [&](int s) { return s * p.seg_len; };
  auto seg_size = [&](int s) { return (uint32_t)(min((s + 1) * p.seg_len, p.nc) - s * p.seg_len); };
  // counters are indexed by the segment of the sequence (launches start on
  // a segment boundary: a window of the pipelined schedule)
  const int seg0 = p.seg_len > 0 ? p.t0 / kChunk / p.seg_len : 0;
  auto seg_done = [&](int s) { return p.done + ((int64_t)(seg0 + s) * p.B * p.H + bh); };
  int* gave_up = reinterpret_cast<int*>(lds + L::FLAG);
  int wseg = 0;  // segments waited for (pipelined schedule); uniform
  if (n_seg > 0) {
    const int first = min(1, p.nc - 1);
    while (wseg < n_seg && seg_start(wseg) <= first) ++wseg;
  }
  bool poison = false;
  if (p.done != nullptr) {
    if (wave == L::NCW) {
      bool ok = true;
      if (n_seg == 0) {
        ok = wait_records(p.done + bh, (uint32_t)p.nc);
      } else {
        for (int s = 0; s < wseg && ok; ++s) ok = wait_records(seg_done(s), seg_size(s));
      }
      if (lane == 0) *gave_up = ok ? 0 : 1;
      if (!ok && lane == 0) raise_status(p.status, kStatusWaitGaveUp);
    }
    __syncthreads();
    poison = *gave_up != 0;
  }

  if (wave < L::NCW) {
    scan_compute_waves<T, D, L>(p, lds, wave, lane, b, h, cb);
  } else {
    // ======================= helper waves =======================
    constexpr int NH = L::NH, VPR = L::VPR;
    const int hid = tid - 64 * L::NCW;
    const bool gated = p.y != nullptr;
    const T* vin = static_cast<const T*>(p.v);
    const T* gin = static_cast<const T*>(p.gate);  // staged only when gated

    // LDS offsets of this thread's units (loop invariant).  Part A and the gate
    // slab split evenly over the helper threads; part B's last units are
    // clamped (a few threads load and store the last unit twice, harmlessly),
    // so that every load and store below is unconditional.
    static_assert(L::A_REC % NH == 0 && L::SLAB_UNITS % NH == 0, "part A and slabs must split evenly");
    constexpr int AR = L::A_REC / NH;  // record steps of part A; the rest is V
    int lofA[L::PA], lofB[L::PB], lofG[L::PG];
#pragma unroll
    for (int i = 0; i < L::PA; ++i) {
      const int u = hid + NH * i;
      lofA[i] = (i < AR) ? lds_offset_of_unit<L, D>(u)
                         : L::VS + ((u - L::A_REC) / VPR) * L::PV + ((u - L::A_REC) % VPR) * 16;
    }
#pragma unroll
    for (int i = 0; i < L::PB; ++i) lofB[i] = lds_offset_of_unit<L, D>(L::A_REC + min(hid + NH * i, L::B_UNITS - 1));
#pragma unroll
    for (int i = 0; i < L::PG; ++i) {
      const int u = hid + NH * i;
      lofG[i] = L::GS + (u / VPR) * L::PV + (u % VPR) * 16;  // + the slab of the chunk (split)
    }
    u32x4 stA[L::PA], stB[L::PB], stG[L::PG];
    // Every byte staged here is read once.  Loads are non-temporal, except
    // the records of the split workgroup, whose other half reads the same
    // record through the shared L2 (measured, K3 layer on the pipelined
    // schedule: 4.57 -> 4.31 ms; with non-temporal stores of y as well it
    // slows to 4.94).
    constexpr bool kStreamRec = NS == 1;
    auto rec_ptr = [&](int c) { return p.ws.base + (bh * p.nc + c) * p.ws.rec_bytes; };
    // `poison`: the records never became complete (staged values become NaN)
    auto last_row = [&](int c) { return min(kChunk, p.T - (p.t0 + c * kChunk)) - 1; };
    // part A of chunk c: qg, kg and the V slab (rows past the end are clamped)
    auto load_A = [&](int c) {
      const u32x4* rp = reinterpret_cast<const u32x4*>(rec_ptr(c));
      const T* v0 = vin + head_base + cb + (int64_t)(p.t0 + c * kChunk) * tok_stride;
      const int last = last_row(c);
#pragma unroll
      for (int i = 0; i < L::PA; ++i) {
        const int u = hid + NH * i;
        if (i < AR) {
          stA[i] = load16<kStreamRec>(rp + u);
        } else if (vin != nullptr) {
          const int vu = u - L::A_REC;
          stA[i] = load16<true>(reinterpret_cast<const u32x4*>(v0 + min(vu / VPR, last) * tok_stride) + vu % VPR);
        } else {  // no V: V = 0
          stA[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      if (poison)
#pragma unroll
        for (int i = 0; i < L::PA; ++i) stA[i] = u32x4{kPoison, kPoison, kPoison, kPoison};
    };
    auto commit_A = [&](int c) {
      const int last = last_row(c);
#pragma unroll
      for (int i = 0; i < L::PA; ++i) {
        u32x4 x = stA[i];
        if (i >= AR) {  // V rows past the end are written as zeros
          const bool zero = (hid + NH * i - L::A_REC) / VPR > last;
#pragma unroll
          for (int w = 0; w < 4; ++w) x[w] = zero ? 0u : x[w];
        }
        *reinterpret_cast<u32x4*>(lds + lofA[i]) = x;
      }
    };
    auto load_B = [&](int c) {
      const u32x4* rp = reinterpret_cast<const u32x4*>(rec_ptr(c)) + L::A_REC;
#pragma unroll
      for (int i = 0; i < L::PB; ++i) stB[i] = load16<kStreamRec>(rp + min(hid + NH * i, L::B_UNITS - 1));
      if (poison)
#pragma unroll
        for (int i = 0; i < L::PB; ++i) stB[i] = u32x4{kPoison, kPoison, kPoison, kPoison};
    };
    static_assert((L::RU.tb - L::RU.kdt) % NH == 0, "Kd^T units fill whole steps");
    auto commit_B = [&]() {
#pragma unroll
      for (int i = 0; i < L::PB; ++i) {
        if (i < L::KDT_STEPS) {  // Kd^T: two 8-byte pieces, 16 rows apart
          *reinterpret_cast<uint2*>(lds + lofB[i]) = uint2{stB[i][0], stB[i][1]};
          *reinterpret_cast<uint2*>(lds + lofB[i] + L::KDT_SECOND) = uint2{stB[i][2], stB[i][3]};
        } else {
          *reinterpret_cast<u32x4*>(lds + lofB[i]) = stB[i];
        }
      }
    };
    auto load_G = [&](int c) {
      const T* g0 = gin + head_base + cb + (int64_t)(p.t0 + c * kChunk) * tok_stride;
      const int last = last_row(c);
#pragma unroll
      for (int i = 0; i < L::PG; ++i) {
        const int u = hid + NH * i;
        stG[i] = load16<true>(reinterpret_cast<const u32x4*>(g0 + min(u / VPR, last) * tok_stride) + u % VPR);
      }
    };
    constexpr int GSLAB = 64 * L::PV;  // bytes of one gate slab
    auto commit_G = [&](int c) {      // gate logits of chunk c into its slab
#pragma unroll
      for (int i = 0; i < L::PG; ++i) *reinterpret_cast<u32x4*>(lds + lofG[i] + (c % L::NOT) * GSLAB) = stG[i];
    };

    // epilogue role: row er, columns ec .. ec + EC - 1 of the workgroup's;
    // gate logits from the slab of the chunk
    using Epi = GateEpilogue<T, D, OUT_F32, NH, false, L::DV>;
    static_assert(Epi::TPR == L::TPR && Epi::EC == L::EC, "epilogue mapping");
    Epi epi;
    epi.init(p, h, hid, cb);
    auto tile_of = [&](int c) {
      return reinterpret_cast<const float*>(lds + L::OT) + (c % L::NOT) * (64 * L::PO);
    };
    auto getg_of = [&](int c) {
      const char* gs = lds + L::GS + (c % L::NOT) * GSLAB + epi.er * L::PV + epi.ec * L::ES;
      return [gs](int q) { return *reinterpret_cast<const u32x4*>(gs + 16 * q); };
    };
    auto epilogue = [&](int c, auto check_rows) {
      epi.template run<decltype(check_rows)::value, L::PO>(p, h, head_base, p.t0 + c * kChunk, tile_of(c), getg_of(c));
    };
    // NS = 2: the row sums of squares of chunk c go through the ring
    // xchg[((b H + h) 2 + half) 4 + c % 4][64] of 8-byte (value, tag) words
    const bool row_lead = (hid % L::TPR) == 0;  // one thread per row publishes
    auto xslot = [&](int hf, int c) {
      return p.xchg + (((bh * 2 + hf) * 4 + (c & 3)) * 64 + epi.er);
    };
    // tag: the chunk's index in the sequence plus one (segments of one call
    // share the ring; the launch before the call's first scan zeroes it)
    auto tag_of = [&](int c) { return (uint32_t)(p.t0 / kChunk + c + 1); };
    auto publish_ss = [&](int c, float ss) {
      if (row_lead)
        __hip_atomic_store(xslot(half, c), (uint64_t)__float_as_uint(ss) | ((uint64_t)tag_of(c) << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto peek_ss = [&](int c) {
      return __hip_atomic_load(xslot(half ^ 1, c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // the other half's sum of squares of chunk c (its word already read once
    // into w); bounded wait, NaN when it never arrives
    auto other_ss = [&](int c, uint64_t w) {
      for (int spin = 0; (uint32_t)(w >> 32) != tag_of(c); ++spin) {
        if (spin >= kCountSpinLimit) {
          raise_status(p.status, kStatusWaitGaveUp);
          return __uint_as_float(kPoison);
        }
        __builtin_amdgcn_s_sleep(2);
        w = peek_ss(c);
      }
      return __uint_as_float((uint32_t)w);
    };
    float ss_last = 0.f, ss_prev = 0.f;  // own half sums of the last two chunks split_first saw
    auto split_first = [&](int c, auto check_rows) {  // o and the half sums of chunk c
      const float ss = epi.template half_ss<decltype(check_rows)::value, L::PO>(p, head_base, p.t0 + c * kChunk,
                                                                             tile_of(c));
      ss_prev = ss_last;
      ss_last = ss;
      if (gated) publish_ss(c, ss);
    };
    // y of chunk c from the own half `mine` and the other half's word w
    auto split_second = [&](int c, float mine, uint64_t w, auto check_rows) {
      if (decltype(check_rows)::value && epi.er >= p.T - (p.t0 + c * kChunk)) return;
      const float ss = mine + other_ss(c, w);
      epi.template split_y<false, L::PO>(p, h, head_base, p.t0 + c * kChunk, tile_of(c), getg_of(c), ss);
    };

    // Loads past the last chunk are clamped to it (their commits land where
    // nobody reads any more), so the steady state has no branches.
    const int cl = p.nc - 1;
    // prologue: part A of chunk 0 into LDS; part B of chunk 0, part A of
    // chunk 1 and the gate logits of chunk 0 into registers
    load_A(0);
    load_B(0);
    commit_A(0);
    load_A(min(1, cl));
    if (gated) load_G(0);
    __syncthreads();
    for (int c = 0; c < p.nc; ++c) {
      // pipelined schedule: chunk c + 2 (loaded in the second half) opens a
      // segment.  Its counter is read at the start of the half, so that the
      // read's latency overlaps the half's work; only a segment not yet
      // complete then needs the bounded wait.  The step also publishes this
      // head's progress for the producer's pacing.
      const bool opens = wseg < n_seg && c + 2 <= cl && c + 2 == seg_start(wseg);
      uint32_t probe = 0;
      if (wave == L::NCW) {
        if (p.progress != nullptr && lane == 0)
          __hip_atomic_store(p.progress + bh, (uint32_t)(p.t0 / kChunk + c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (opens && !poison) probe = __hip_atomic_load(const_cast<uint32_t*>(seg_done(wseg)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // split: the other half's sums of chunk c - 2, read early
      uint64_t wprev = 0;
      if (NS == 2 && gated && c > 1) wprev = peek_ss(c - 2);
      // first half of step c: the compute waves read part A of chunk c
      commit_B();                                        // part B of chunk c
      load_B(min(c + 1, cl));
      if constexpr (NS == 1) {
        if (c > 0) epilogue(c - 1, std::false_type{});   // tile and gate logits of chunk c - 1
      } else {
        if (c > 0) split_first(c - 1, std::false_type{});                       // o and half sums of chunk c - 1
        if (gated && c > 1) split_second(c - 2, ss_prev, wprev, std::false_type{});  // y of chunk c - 2
      }
      if (opens && wave == L::NCW && !poison) {
        const uint32_t need = seg_size(wseg);
        bool ok = true;
        if (__builtin_amdgcn_readfirstlane(probe) >= need)
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        else
          ok = wait_records(seg_done(wseg), need);
        if (lane == 0) *gave_up = ok ? 0 : 1;
        if (!ok && lane == 0) raise_status(p.status, kStatusWaitGaveUp);
      }
      __syncthreads();
      if (opens) {
        ++wseg;
        poison = poison || *gave_up != 0;
      }
      // second half: the compute waves read part B of chunk c and write tile c
      commit_A(min(c + 1, cl));
      if (gated) commit_G(c);                            // gate logits of chunk c
      load_A(min(c + 2, cl));
      if (gated) load_G(min(c + 1, cl));
      __syncthreads();
    }
    if constexpr (NS == 1) {
      epilogue(cl, std::true_type{});
    } else {
      split_first(cl, std::true_type{});
      if (gated) {
        if (cl > 0) split_second(cl - 1, ss_prev, peek_ss(cl - 1), std::false_type{});
        split_second(cl, ss_last, peek_ss(cl), std::true_type{});
      }
    }
  }
}

template <typename T, int D>
static void launch_scan_t(const ScanParams& p, hipStream_t s) {
  using W = WsLds<T, D>;
  if constexpr (W::FITS) {
    if constexpr (split_supported(sizeof(T), D)) {
      using W2 = WsLds<T, D, 2>;
      static_assert(W2::FITS, "the split workgroup fits");
      if (p.nsplit == 2) {
        const dim3 grid((unsigned)(16 * ((p.B * p.H + 7) / 8)));
        if (p.out_f32)
          hipLaunchKernelGGL((kda_scan_ws_kernel<T, D, true, 2>), grid, dim3(W2::NT), 0, s, p);
        else
          hipLaunchKernelGGL((kda_scan_ws_kernel<T, D, false, 2>), grid, dim3(W2::NT), 0, s, p);
        return;
      }
    }
    if (p.out_f32)
      hipLaunchKernelGGL((kda_scan_ws_kernel<T, D, true, 1>), dim3(p.H, p.B), dim3(W::NT), 0, s, p);
    else
      hipLaunchKernelGGL((kda_scan_ws_kernel<T, D, false, 1>), dim3(p.H, p.B), dim3(W::NT), 0, s, p);
  } else {
    hipLaunchKernelGGL((kda_scan_serial_kernel<T, D>), dim3(p.H, p.B), dim3(4 * D), 0, s, p);
  }
}

hipError_t launch_scan(const ScanParams& p, int D, int in_f32, hipStream_t s) {
  if (in_f32) {
    if (D == 64) launch_scan_t<float, 64>(p, s);
    else launch_scan_t<float, 128>(p, s);
  } else {
    if (D == 64) launch_scan_t<uint16_t, 64>(p, s);
    else launch_scan_t<uint16_t, 128>(p, s);
  }
  return hipGetLastError();
}

}  // namespace kda
