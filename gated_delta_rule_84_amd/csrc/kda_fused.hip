// Fused forward: one workgroup per (head, batch) runs the whole chunked
// forward of its head in one launch, and the chunk records never leave the
// CU.  D / 32 compute waves run the state scan's MFMA chain on chunk c (the
// same code as the scan kernel, over an LDS image of the record) while four
// producer waves -- one per 16-token sub-tile -- run the intra-chunk steps of
// chunk c + 1 straight into that image, stage V, and turn chunk c - 1's output
// tile into o / y.
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3), sections 2.1-2.3; the arithmetic is
// that of the intra-chunk steps and of the scan (kda_intra_core.hpp,
// kda_scan_core.hpp), so the results equal those of the two-kernel path bit
// for bit.
//
// Chunk step c (the compute waves' two halves, split by the workgroup
// barriers M and E):
//   compute, first half  -- part A of chunk c (qg, kg) and the V slab
//   producers, first half -- distance levels of chunk c's UT inverse, tb,
//                            Kd^T, Tril(A_qk), Gamma_last (part B of chunk c);
//                            o / y of chunk c - 1 (its gate logits loaded at
//                            the start of the half); V of chunk c + 1 into
//                            registers
//   -- M --
//   compute, second half -- part B of chunk c; output tile of chunk c
//   producers, second half -- intra-chunk steps of chunk c + 1 up to the
//                            diagonal blocks of T (part A of chunk c + 1 into
//                            the image), V of chunk c + 1 into LDS; q, k, z,
//                            beta of chunk c + 2 into registers
//   -- E --
// The producers synchronise among themselves between intra-chunk steps with
// an LDS counter (the compute waves are not held by it).  The V slab's space
// holds, between two V slabs, the column factors, anchor rows and totals of
// the chunk being produced.
#include "kda_intra_core.hpp"
#include "kda_scan_core.hpp"

namespace kda {

template <typename T, int D>
struct FusedLds {
  static constexpr int ES = sizeof(T);
  static constexpr int NCW = D / 32;           // compute waves
  static constexpr int NPW = 4;                // producer waves
  static constexpr int NT = 64 * (NCW + NPW);  // threads
  static constexpr int NP = 64 * NPW;          // producer threads
  static constexpr int RS = sizeof(typename RecOps<T>::Elem);  // record element
  static_assert(RS == ES, "one row pitch for the record and the V slab");
  static constexpr int PQ = D * ES + 16;       // row pitch of qg / kg / V slab (bytes)
  static constexpr int PV = PQ;                // of the V slab, as the scan's compute waves read it
  static constexpr int NCT = 2;                // 16-column tiles per compute wave
  static constexpr int NOT = 1;                // output tiles
  static constexpr int PK = 64 * RS + 16;      // row pitch of kdt / tb / aq (bytes)
  static constexpr int PO = D + 4;             // output tile row pitch (floats)
  // record image read by the compute waves
  static constexpr int QG = 0;
  static constexpr int KG = QG + 64 * PQ;
  static constexpr int KDT = KG + 64 * PQ;
  static constexpr int TB = KDT + D * PK;
  static constexpr int AQ = TB + 64 * PK;
  static constexpr int GAM = AQ + 64 * PK;
  static constexpr int VS = GAM + 4 * D;       // V slab [64][PQ]
  static constexpr int OT = VS + 64 * PQ;      // output tile [64][PO] fp32
  // intra-chunk work areas (producers only)
  static constexpr int ET = OT + 64 * PO * 4;  // [6][D]
  static constexpr int EB = ET + 6 * D * 4;    // [4][D]
  static constexpr int EL = EB + 4 * D * 4;    // [4][D]
  static constexpr int BETA = EL + 4 * D * 4;  // [64]
  static constexpr int GAMS = BETA + 64 * 4;   // Gamma_last of the chunk being produced [D]
  static constexpr int TM = GAMS + 4 * D;      // T [64][68] fp32
  static constexpr int CTR = TM + 64 * 68 * 4; // producer barrier counter
  static constexpr int BYTES = CTR + 16;
  // inside the V slab's space (free between two V slabs): the column factors,
  // then the anchor rows and totals behind them (the anchors are still read
  // while the column factors are written)
  static constexpr int KP = D + 16 / ES;
  static constexpr int KC = VS;                                  // [48][KP] elements of T
  static constexpr int LOC7 = VS + ((48 * KP * ES + 15) / 16) * 16;  // [4][D]
  static constexpr int TOT = LOC7 + 4 * D * 4;                   // [4][D]
  static constexpr int VPR = D * ES / 16;      // 16-byte units per V row
  static constexpr int VU = 64 * VPR / NP;     // V units per producer thread
  static_assert(TOT + 4 * D * 4 <= VS + 64 * PQ, "KC, loc7 and tot must fit in the V slab's space");
  static_assert(64 * VPR % NP == 0, "V slab must split evenly");
  static constexpr bool FITS = ES == 2 && BYTES <= 160 * 1024;
};

// Barrier among the producer waves only.  Each producer wave adds one to an
// LDS counter once its own LDS writes have completed, then waits until all
// waves of this round have arrived (the count reaches `target`).  All
// producer waves pass the same sequence of these barriers and of the
// workgroup barriers, so none waits on a wave held elsewhere.  The wait is
// bounded; should it ever run out, the wave stops waiting at every later
// barrier too (results would be wrong, but the kernel still completes).
template <int NPW>
__device__ __forceinline__ void producer_sync(unsigned* ctr, unsigned& target, bool& broken) {
  target += NPW;
  __builtin_amdgcn_sched_barrier(0);   // no instruction moves across the barrier
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes have landed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (!broken) {
    int spin = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
      if (++spin > (1 << 20)) {
        broken = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

template <typename T, int D, bool OUT_F32>
__global__ __launch_bounds__((FusedLds<T, D>::NT), 1) void kda_fused_kernel(const IntraParams ip, const ScanParams p) {
  using L = FusedLds<T, D>;
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x, b = blockIdx.y;
  unsigned* ctr = reinterpret_cast<unsigned*>(lds + L::CTR);
  if (tid == 0) *ctr = 0u;
  __syncthreads();

  if (wave < L::NCW) {
    scan_compute_waves<T, D, L>(p, lds, wave, lane, b, h);
    return;
  }

  // ======================= producer waves =======================
  using Core = IntraCore<T, D, L::PQ / L::ES, L::PK / L::ES>;
  // the epilogue runs on 2 D producer threads: the thread mapping, and so the
  // order of the RMS sums, of the scan kernel's helper waves
  using Epi = GateEpilogue<T, D, OUT_F32, 2 * D, true>;
  static_assert(2 * D <= L::NP, "epilogue threads");
  static_assert(Core::KP == L::KP, "column factor pitch");
  int pt = tid - 64 * L::NCW;  // producer thread
  const IntraScratch<T> s{reinterpret_cast<float*>(lds + L::LOC7), reinterpret_cast<float*>(lds + L::TOT),
                          reinterpret_cast<float*>(lds + L::ET),   reinterpret_cast<float*>(lds + L::EB),
                          reinterpret_cast<float*>(lds + L::EL),   reinterpret_cast<float*>(lds + L::BETA),
                          reinterpret_cast<T*>(lds + L::KC),       reinterpret_cast<float*>(lds + L::TM)};
  T* qg = reinterpret_cast<T*>(lds + L::QG);
  T* kg = reinterpret_cast<T*>(lds + L::KG);
  T* kdt = reinterpret_cast<T*>(lds + L::KDT);
  T* tb = reinterpret_cast<T*>(lds + L::TB);
  T* aq = reinterpret_cast<T*>(lds + L::AQ);
  float* gam = reinterpret_cast<float*>(lds + L::GAM);
  float* gams = reinterpret_cast<float*>(lds + L::GAMS);
  const float* otile = reinterpret_cast<const float*>(lds + L::OT);
  const int64_t tok_stride = token_stride(p.head_first, p.H, D);
  const int64_t head_base = token_base(p.head_first, b, h, p.T, p.H, D);
  const int nc = p.nc;
  auto nvalid_of = [&](int c) { return min(kChunk, p.T - c * kChunk); };

  unsigned target = 0;
  bool broken = false;
  auto psync = [&]() { producer_sync<L::NPW>(ctr, target, broken); };

  Core ic;
  ic.init(wave - L::NCW, lane);
  Epi epi;
  epi.init(p, h, pt);

  // V slab of chunk c: into registers, then into LDS with rows past the end zeroed
  u32x4 vst[L::VU];
  auto load_V = [&](int c) {
    const T* v0 = static_cast<const T*>(p.v) + head_base + (int64_t)(c * kChunk) * tok_stride;
    const int last = nvalid_of(c) - 1;
#pragma unroll
    for (int i = 0; i < L::VU; ++i) {
      const int u = pt + L::NP * i;
      vst[i] = p.v != nullptr ? reinterpret_cast<const u32x4*>(v0 + min(u / L::VPR, last) * tok_stride)[u % L::VPR]
                              : u32x4{0u, 0u, 0u, 0u};  // no V: V = 0
    }
  };
  auto commit_V = [&](int c) {
    const int last = nvalid_of(c) - 1;
#pragma unroll
    for (int i = 0; i < L::VU; ++i) {
      const int u = pt + L::NP * i;
      u32x4 x = vst[i];
      const bool zero = u / L::VPR > last;
#pragma unroll
      for (int w = 0; w < 4; ++w) x[w] = zero ? 0u : x[w];
      *reinterpret_cast<u32x4*>(lds + L::VS + (u / L::VPR) * L::PQ + (u % L::VPR) * 16) = x;
    }
  };
  u32x4 gst[Epi::NG];  // gate logits of the chunk whose tile is turned into o / y
  auto getg = [&](int q) { return gst[q]; };
  const bool gated = p.y != nullptr;
  const bool epi_thread = pt < 2 * D;  // whole waves

  // Intra-chunk steps of chunk c up to the diagonal blocks of T; part A of
  // chunk c goes into the image.  q, k, z, beta of chunk c are in registers.
  auto produce_front = [&]() {
    ic.prefix(ip, h, s);
    psync();  // anchors and totals
    Core::template tables<L::NP>(pt, s, gams);
    psync();  // tables built; the totals are dead
    ic.factors(s, qg, kg);
    psync();  // column factors and L_ii stages
    ic.offdiag(s);
    ic.solve(s);
    psync();  // the column factors are dead; every T_ii is in LDS
  };
  // The rest of the chunk: off-diagonal blocks of T by distance, then part B.
  auto produce_back = [&]() {
    ic.level(1, s);
    psync();
    ic.level(2, s);
    psync();
    ic.level(3, s);
    psync();
    Core::template tb_pass<L::NP>(pt, s, tb);
    ic.store_kd(kdt);
    ic.store_aq(aq);
    if (pt < D) gam[pt] = gams[pt];
  };

  // prologue: chunk 0 up to its part A and V slab; q, k, z, beta of chunk 1
  ic.load(ip, b, h, 0, nvalid_of(0));
  load_V(0);
  produce_front();
  commit_V(0);
  if (nc > 1) ic.load(ip, b, h, kChunk, nvalid_of(1));
  __syncthreads();  // part A of chunk 0 staged

  // Per-lane index arithmetic is redone in each half from an opaque copy of
  // the lane id, so that the compiler cannot hoist the (many, 64-bit) per-lane
  // addresses out of the loop and keep them live across it.
  auto refresh = [&]() {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    ic.init(wave - L::NCW, ln);
    epi.init(p, h, 64 * (wave - L::NCW) + ln);
    pt = 64 * (wave - L::NCW) + ln;
  };
  for (int c = 0; c < nc; ++c) {
    // first half of step c
    refresh();
    if (c > 0 && gated && epi_thread) epi.load_gate(p, head_base, (c - 1) * kChunk, gst);
    if (c + 1 < nc) load_V(c + 1);
    produce_back();  // part B of chunk c
    if (c > 0 && epi_thread) epi.template run<false, L::PO>(p, h, head_base, (c - 1) * kChunk, otile, getg);
    __syncthreads();  // M: part A of chunk c consumed, part B staged
    // second half of step c
    refresh();
    if (c + 1 < nc) {
      produce_front();  // part A of chunk c + 1
      commit_V(c + 1);
      if (c + 2 < nc) ic.load(ip, b, h, (c + 2) * kChunk, nvalid_of(c + 2));
    }
    __syncthreads();  // E: part B of chunk c consumed; tile c, part A of chunk c + 1 staged
  }
  if (!epi_thread) return;
  if (gated) epi.load_gate(p, head_base, (nc - 1) * kChunk, gst);
  epi.template run<true, L::PO>(p, h, head_base, (nc - 1) * kChunk, otile, getg);
}

template <typename T, int D>
static hipError_t launch_fused_t(const IntraParams& ip, const ScanParams& p, hipStream_t s) {
  using L = FusedLds<T, D>;
  if constexpr (L::FITS) {
    if (p.out_f32)
      hipLaunchKernelGGL((kda_fused_kernel<T, D, true>), dim3(p.H, p.B), dim3(L::NT), 0, s, ip, p);
    else
      hipLaunchKernelGGL((kda_fused_kernel<T, D, false>), dim3(p.H, p.B), dim3(L::NT), 0, s, ip, p);
    return hipGetLastError();
  } else {
    return hipErrorInvalidConfiguration;
  }
}

bool fused_supported(int D, int in_f32) { return !in_f32 && (D == 64 || D == 128); }

hipError_t launch_fused(const IntraParams& ip, const ScanParams& p, int D, int in_f32, hipStream_t s) {
  if (!fused_supported(D, in_f32)) return hipErrorInvalidConfiguration;
  return D == 64 ? launch_fused_t<uint16_t, 64>(ip, p, s) : launch_fused_t<uint16_t, 128>(ip, p, s);
}

}  // namespace kda
