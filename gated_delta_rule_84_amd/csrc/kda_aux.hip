// State import / export and the pre-pass diagnostic.
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3), section 2.2 (decay map, used by the
// pre-pass).
#include "kda_chunk_prologue.hpp"

namespace kda {

// ---- state import / export / zero: one workgroup per (n, h) ----------------
template <int D>
__global__ __launch_bounds__(256) void kda_state_io_kernel(const StateIoParams p) {
  __shared__ float tile[32][33];
  const int h = blockIdx.x, n = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t slot = (p.slot != nullptr) ? (int64_t)p.slot[n] : (int64_t)n;
  if (slot < 0 || slot >= p.n_slots) {  // uniform over the workgroup: nothing is touched
    if (tid == 0) raise_status(p.status, kFlagBadSlot);
    return;
  }
  float* pool = p.pool + (slot * p.H + h) * D * D;
  float* user = (p.user != nullptr) ? p.user + ((int64_t)n * p.H + h) * D * D : nullptr;
  // Same layout: a copy of the head's D x D floats in 16-byte vectors (each
  // element is read and written by the same thread, so an in-place call is
  // still exact); element by element when a pointer is only 4-byte aligned.
  // Measured on the decode pool (256 x 96 states): 5.3 TB/s against 4.8 TB/s
  // element by element, and 3.7 TB/s with all of a thread's 16 loads issued
  // before its stores; with non-temporal loads and stores (every byte is
  // touched once) 5.6 TB/s.
  constexpr int N4 = D * D / 4 / 256;  // 16-byte vectors per thread
  if (!p.vec16 && (p.op == 0 || !p.transpose)) {
    if (p.op == 0)
      for (int i = tid; i < D * D; i += 256) pool[i] = 0.f;
    else if (p.op == 1)
      for (int i = tid; i < D * D; i += 256) pool[i] = user[i];
    else
      for (int i = tid; i < D * D; i += 256) user[i] = pool[i];
    return;
  }
  if (p.op == 0) {
    float4* d4 = reinterpret_cast<float4*>(pool);
#pragma unroll
    for (int j = 0; j < N4; ++j) d4[tid + 256 * j] = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  if (!p.transpose) {
    const u32x4* s4 = reinterpret_cast<const u32x4*>(p.op == 1 ? user : pool);
    u32x4* d4 = reinterpret_cast<u32x4*>(p.op == 1 ? pool : user);
#pragma unroll 4
    for (int j = 0; j < N4; ++j) __builtin_nontemporal_store(__builtin_nontemporal_load(s4 + tid + 256 * j), d4 + tid + 256 * j);
    return;
  }
  // transposed user layout [d_v][d_k]: 32x32 tiles through LDS
  const float* src = (p.op == 1) ? user : pool;
  float* dst = (p.op == 1) ? pool : user;
  const int tx = tid & 31, ty = tid >> 5;  // 32 x 8
  for (int bi = 0; bi < D; bi += 32)
    for (int bj = 0; bj < D; bj += 32) {
      for (int r = ty; r < 32; r += 8) tile[r][tx] = src[(bi + r) * D + bj + tx];
      __syncthreads();
      for (int r = ty; r < 32; r += 8) dst[(bj + r) * D + bi + tx] = tile[tx][r];
      __syncthreads();
    }
}

hipError_t launch_state_io(const StateIoParams& p, int D, hipStream_t s) {
  const dim3 grid(p.H, p.n), block(256);
  if (D == 64) hipLaunchKernelGGL((kda_state_io_kernel<64>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((kda_state_io_kernel<128>), grid, block, 0, s, p);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void kda_copy_state_kernel(const float* src, float* dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = (src != nullptr) ? src[i] : 0.f;
}

hipError_t launch_copy_state(const float* src, float* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(kda_copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

// ---- pre-pass diagnostic: chunk-local cumulative log-decay and norms -------
// Runs the same device routines as the intra-chunk kernel's prologue: wave i
// forms sub-tile i's decay prefix in registers; the sub-tile totals are then
// added up across the chunk through LDS.
template <typename T, int D, bool SP>
__global__ __launch_bounds__(256) void kda_prepass_kernel(const PrepassParams p) {
  constexpr int KS = D / 32;
  __shared__ __attribute__((aligned(16))) float tot[4 * D];
  using R8 = Run8<T>;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int tok0 = c * kChunk;
  const int nvalid = min(kChunk, p.T - tok0);
  const int64_t tok_stride = (int64_t)p.H * D;
  const int64_t row0 = ((int64_t)b * p.T + tok0) * p.H * D + (int64_t)h * D;
  const int r = 16 * wave + n;
  const bool rvalid = r < nvalid;
  const int64_t rowp = row0 + min(r, nvalid - 1) * tok_stride;
  typename R8::Raw qraw[KS], kraw[KS], zraw[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    qraw[kk] = R8::load(static_cast<const T*>(p.q) + rowp, kk, g4);
    kraw[kk] = R8::load(static_cast<const T*>(p.k) + rowp, kk, g4);
    zraw[kk] = R8::load(static_cast<const T*>(p.z) + rowp, kk, g4);
  }
  float P[KS][8];
  subtile_decay_prefix<T, KS, SP>(zraw, p.A[h], p.g_min, 1.0f, rvalid, P);
  if (n == 15)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) put_run8(tot + wave * D, kk, g4, P[kk]);
  const float rq = row_inv_norm<T, KS>(qraw, p.l2norm, p.l2_eps);
  const float rk = row_inv_norm<T, KS>(kraw, p.l2norm, p.l2_eps);
  __syncthreads();
  if (rvalid) {
    float* Grow = p.G + row0 + r * tok_stride;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      float off[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int w = 0; w < wave; ++w) {
        float t[8];
        lds_run8(tot + w * D, kk, g4, t);
#pragma unroll
        for (int j = 0; j < 8; ++j) off[j] += t[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) off[j] += P[kk][j];
      put_run8(Grow, kk, g4, off);
    }
    if (g4 == 0) {
      const int64_t ri = ((int64_t)b * p.T + tok0 + r) * p.H + h;
      p.rq[ri] = rq;
      p.rk[ri] = rk;
    }
  }
}

template <bool SP>
static void launch_prepass_t(const PrepassParams& p, int D, int in_f32, hipStream_t s) {
  const dim3 grid((p.T + kChunk - 1) / kChunk, p.H, p.B), block(256);
  if (in_f32) {
    if (D == 64) hipLaunchKernelGGL((kda_prepass_kernel<float, 64, SP>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((kda_prepass_kernel<float, 128, SP>), grid, block, 0, s, p);
  } else {
    if (D == 64) hipLaunchKernelGGL((kda_prepass_kernel<uint16_t, 64, SP>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((kda_prepass_kernel<uint16_t, 128, SP>), grid, block, 0, s, p);
  }
}

hipError_t launch_prepass(const PrepassParams& p, int D, int in_f32, hipStream_t s) {
  if (p.decay) launch_prepass_t<true>(p, D, in_f32, s);
  else launch_prepass_t<false>(p, D, in_f32, s);
  return hipGetLastError();
}

}  // namespace kda
