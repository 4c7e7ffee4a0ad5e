// Chunk-parallel scan over segments of a sequence (KCP, one GPU's share).
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3), section 10.2: over a segment the state
// map is affine, S_out = M S_in + S~, with M the product of the per-token
// transfers (I - beta_t k_t k_t^T) Diag(alpha_t) and S~ the state reached
// from S = 0; pairs compose associatively, (M2, S2) o (M1, S1) =
// (M2 M1, S2 + M2 S1).  Here the pairs of all segments come from the forward
// itself (M: from S_in = I with V = 0; S~: from S_in = 0), and this kernel
// folds them along each sequence into every segment's entry state:
//     S_in[0] = S0,  S_in[p + 1] = M[p] S_in[p] + S~[p].
#include "kda_common.hpp"
#include "kda_params.hpp"

namespace kda {

namespace {

// One workgroup per (h, b), 256 threads.  The running state is kept in LDS
// (D x (D + 1) fp32).  Thread t owns column t % D and the RPT = D^2 / 256
// rows starting at (t / D) RPT (the same rows for a whole wave, so the
// entries of M it needs are wave-uniform loads); it accumulates over k in a
// fixed order, fp32.
template <int D>
__global__ __launch_bounds__(256) void kda_kcp_fold_kernel(const float* M, const float* St, const float* S0,
                                                           float* Sin, int P, int H) {
  constexpr int RPT = D * D / 256;  // rows per thread (one column each)
  __shared__ float S[D][D + 1];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int j = tid % D;
  const int r0 = __builtin_amdgcn_readfirstlane((tid / D) * RPT);
  const int64_t DD = (int64_t)D * D;
  const int64_t stride_p = (int64_t)H * DD;  // between segments of one sequence
  const int64_t first = ((int64_t)b * P * H + h) * DD;  // segment 0 of (b, h)

  // S_in[0] = S0 (or zero)
  const float* s0 = S0 != nullptr ? S0 + ((int64_t)b * H + h) * DD : nullptr;
  float* out0 = Sin + first;
  for (int i = tid; i < D * D; i += 256) {
    const float v = s0 != nullptr ? s0[i] : 0.0f;
    S[i / D][i % D] = v;
    out0[i] = v;
  }
  __syncthreads();
  for (int p = 0; p + 1 < P; ++p) {
    const float* m = M + first + p * stride_p;
    const float* st = St + first + p * stride_p;
    float acc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) acc[r] = 0.0f;
    for (int k = 0; k < D; ++k) {
      const float skj = S[k][j];
#pragma unroll
      for (int r = 0; r < RPT; ++r) acc[r] = __builtin_fmaf(m[(int64_t)(r0 + r) * D + k], skj, acc[r]);
    }
    __syncthreads();  // every thread has read S
    float* out = Sin + first + (p + 1) * stride_p;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const float v = acc[r] + st[(int64_t)(r0 + r) * D + j];
      S[r0 + r][j] = v;
      out[(int64_t)(r0 + r) * D + j] = v;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void kda_identity_states_kernel(float* dst, int64_t n, int D) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t DD = (int64_t)D * D;
  if (i < n * DD) {
    const int64_t e = i % DD;
    dst[i] = (e / D == e % D) ? 1.0f : 0.0f;
  }
}

}  // namespace

hipError_t launch_kcp_fold(const float* M, const float* St, const float* S0, float* Sin, int B, int P, int H, int D,
                           hipStream_t s) {
  const dim3 grid(H, B);
  if (D == 64)
    hipLaunchKernelGGL((kda_kcp_fold_kernel<64>), grid, dim3(256), 0, s, M, St, S0, Sin, P, H);
  else
    hipLaunchKernelGGL((kda_kcp_fold_kernel<128>), grid, dim3(256), 0, s, M, St, S0, Sin, P, H);
  return hipGetLastError();
}

hipError_t launch_identity_states(float* dst, int64_t n, int D, hipStream_t s) {
  const int64_t total = n * D * D;
  if (total > 0)
    hipLaunchKernelGGL(kda_identity_states_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, dst, n, D);
  return hipGetLastError();
}

}  // namespace kda
