// Intra-chunk kernel: workgroups of 4 waves run the intra-chunk steps of
// kda_intra_core.hpp for the launch's (chunk, batch, head) records and write
// each record to the workspace for the state scan.
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3), sections 2.1 and 2.2 (see
// kda_intra_core.hpp for the factorisation and the precision plan).
#include "kda_intra_core.hpp"

namespace kda {

// LDS layout (bytes).  Small per-channel tables first, then the column
// factors of sub-tiles 0..2 (the only ones used as off-diagonal columns) and
// the fp32 UT inverse, row-major.
template <typename T, int D>
struct IntraLds {
  static constexpr int ES = sizeof(T);
  static constexpr int KP = D + 16 / ES;  // KC row pitch (elements)
  static constexpr int LP = 68;           // T row pitch (floats)
  static constexpr int LOC7 = 0;          // prefix at each sub-tile's anchor row  [4][D]
  static constexpr int TOT = LOC7 + 4 * D * 4;   // sub-tile totals              [4][D]
  static constexpr int ET = TOT + 4 * D * 4;     // e^{B_i - B_j}, 6 pairs i > j  [6][D]
  static constexpr int EB = ET + 6 * D * 4;      // e^{B_i}                       [4][D]
  static constexpr int EL = EB + 4 * D * 4;      // e^{G_last - B_i}              [4][D]
  static constexpr int BETA = EL + 4 * D * 4;    // beta                          [64]
  static constexpr int KC = BETA + 64 * 4;       // column factors                [48][KP]
  static constexpr int TM = KC + ((48 * KP * ES + 15) / 16) * 16;  // T          [64][LP]
  static constexpr int BYTES = TM + 64 * LP * 4;
};

// One workgroup (4 waves) per record of the launch, in chunk-major order:
// workgroup item = c B H + b H + h, so that the records of a chunk come out
// together for every head, as the state scan consumes them, and the rows of
// a chunk's q, k, z are read for all heads at once (c counted from the last
// chunk when IntraParams::reverse is set).  In the pipelined
// schedule the launch is paced by the scan's progress (IntraParams::progress).
//
// SP: the unbounded softplus decay (pairwise diagonal blocks, more registers:
// two workgroups per CU).
template <typename T, int D, bool SP>
__global__ __launch_bounds__(256, (sizeof(T) == 2 && !SP ? 3 : 2)) void kda_intra_kernel(const IntraParams p) {
  using L = IntraLds<T, D>;
  using Core = IntraCore<T, D, D, kChunk, SP, true>;  // record in the workspace's unit layout
  static_assert(Core::KP == L::KP && Core::LP == L::LP, "scratch pitches");
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
  const IntraScratch<T> s{reinterpret_cast<float*>(lds + L::LOC7), reinterpret_cast<float*>(lds + L::TOT),
                          reinterpret_cast<float*>(lds + L::ET),   reinterpret_cast<float*>(lds + L::EB),
                          reinterpret_cast<float*>(lds + L::EL),   reinterpret_cast<float*>(lds + L::BETA),
                          reinterpret_cast<T*>(lds + L::KC),       reinterpret_cast<float*>(lds + L::TM)};

  const int tid = threadIdx.x;
  const int bh_n = p.B * p.H;
  const int item = blockIdx.x;
  const int c = p.reverse ? p.nc - 1 - item / bh_n : item / bh_n, bh = item % bh_n;
  const int b = bh / p.H, h = bh % p.H;
  const int tok0 = p.t0 + c * kChunk;
  const int nvalid = min(kChunk, p.T - tok0);
  const int64_t stride = p.rec_stride > 0 ? p.rec_stride : p.nc;
  const int64_t rec = (int64_t)bh * stride + p.rec_c0 + c;
  constexpr RecUnits RU = rec_units((int)sizeof(T), D);
  char* recp = p.ws.base + rec * p.ws.rec_bytes;

  if (p.clear != nullptr)
    for (int64_t w = (int64_t)item * 256 + tid; w < p.clear_words; w += (int64_t)gridDim.x * 256) p.clear[w] = 0;
  if (p.clear_status != nullptr && item == 0 && tid == 0) *p.clear_status = 0;
  const int cg = p.t0 / kChunk + c;  // chunk index in the sequence
  if (p.progress != nullptr && cg % kPaceEvery == 0 && cg > p.lead) {  // uniform: pacing (see IntraParams)
    if (tid == 0) pace(p.progress + bh, (uint32_t)(cg - p.lead), p.pacing_off);
    __syncthreads();
  }
  Core ic;
  ic.init(tid >> 6, tid & 63);
  ic.sink = rec_sink(recp, (int)p.ws.rec_bytes);
  ic.load(p, b, h, tok0, nvalid);
  ic.prefix(p, h, s);
  __syncthreads();
  Core::template tables<256>(tid, s, reinterpret_cast<float*>(recp + 16 * RU.gam), &ic.sink);
  __syncthreads();
  ic.factors(s, reinterpret_cast<T*>(recp + 16 * RU.qg), reinterpret_cast<T*>(recp + 16 * RU.kg));
  ic.store_kd(reinterpret_cast<T*>(recp + 16 * RU.kdt));
  __syncthreads();  // column factors and the L_ii stages are visible
  ic.offdiag(s);
  ic.store_aq(reinterpret_cast<T*>(recp + 16 * RU.aq));
  ic.solve(s);
  __syncthreads();  // every T_ii is in LDS
#pragma unroll
  for (int dist = 1; dist <= 3; ++dist) {
    ic.level(dist, s);
    __syncthreads();
  }
  Core::template tb_pass<256>(tid, s, reinterpret_cast<T*>(recp + 16 * RU.tb), &ic.sink);
  if (p.done != nullptr) {
    // the record's counter: that of its segment of the sequence (one
    // segment if seg_len = 0)
    const int seg = p.seg_len > 0 ? cg / p.seg_len : 0;
    count_record(p.done + (int64_t)seg * bh_n + bh);
  }
}

template <bool SP>
static void launch_intra_t(const IntraParams& p, int D, int in_f32, hipStream_t s) {
  const dim3 grid((unsigned)(p.nc * p.B * p.H)), block(256);
  if (in_f32) {
    if (D == 64) hipLaunchKernelGGL((kda_intra_kernel<float, 64, SP>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((kda_intra_kernel<float, 128, SP>), grid, block, 0, s, p);
  } else {
    if (D == 64) hipLaunchKernelGGL((kda_intra_kernel<uint16_t, 64, SP>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((kda_intra_kernel<uint16_t, 128, SP>), grid, block, 0, s, p);
  }
}

hipError_t launch_intra(const IntraParams& p, int D, int in_f32, hipStream_t s) {
  if (p.nc <= 0) return hipSuccess;
  if (p.decay) launch_intra_t<true>(p, D, in_f32, s);
  else launch_intra_t<false>(p, D, in_f32, s);
  return hipGetLastError();
}

}  // namespace kda
