// Input steps before the KDA core: q, k and v each pass through a ShortConv
// (a depthwise causal convolution over time, W taps per channel) and Swish;
// beta = Sigmoid(beta logit).  The L2Norm of q and k is done by the core.
//
// Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
// (hs-black.github.io/posts/kimi-k3), section 2.1 (ShortConv, Swish and
// L2Norm on q and k; ShortConv and Swish on v; Sigmoid for beta).  The pages
// give neither the convolution's width nor a bias: W is a parameter (1..4),
// and there is no bias.
//
// HBM-bound streaming kernel.  One thread owns 8 consecutive channels (one
// 16-byte vector of bf16) of one stream of one sequence, over a block of
// tokens (128 unless the state is updated in place): it keeps the last W-1
// inputs in registers, loads the
// block's tokens 8 at a time ahead of their use, and accumulates the taps in
// a fixed order (so that results never depend on the blocking).  The W-1
// tokens before a block are re-read (from the sequence, or from the carried
// state before token 0).  A wave covers 512 consecutive channels of one
// token: every load and store is a contiguous 1 KB (bf16).  The block's own
// tokens are loaded and the outputs stored non-temporally (each is touched
// once; measured at the K3 layer's shapes: 1.89 -> 1.84 ms, while either
// alone changes nothing); the few halo tokens re-read by the next block are
// plain loads.
#include "kda_common.hpp"
#include "kda_params.hpp"

namespace kda {

namespace {

template <typename T>
struct Vec8;
template <>
struct Vec8<uint16_t> {
  template <bool STREAM = false>
  static __device__ __forceinline__ void load(const uint16_t* p, float* x) {
    const u32x4 w = load16<STREAM>(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* x) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack2_bf16(x[2 * i], x[2 * i + 1]);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
  }
};
template <>
struct Vec8<float> {
  template <bool STREAM = false>
  static __device__ __forceinline__ void load(const float* p, float* x) {
    const u32x4 a = load16<STREAM>(reinterpret_cast<const u32x4*>(p));
    const u32x4 b = load16<STREAM>(reinterpret_cast<const u32x4*>(p + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(a[i]);
      x[4 + i] = __uint_as_float(b[i]);
    }
  }
  static __device__ __forceinline__ void store(float* p, const float* x) {
    __builtin_nontemporal_store(u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])},
                                reinterpret_cast<u32x4*>(p));
    __builtin_nontemporal_store(u32x4{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])},
                                reinterpret_cast<u32x4*>(p + 4));
  }
};

constexpr int kUnroll = 8;  // tokens loaded ahead of their use

// grid (ceil(C / 2048), token blocks, 3 B): stream s = z % 3 (q, k, v), b = z / 3
template <typename T, int W>
__global__ __launch_bounds__(256) void kda_prep_conv_kernel(const InputPrepParams p) {
  const int s = blockIdx.z % 3, b = blockIdx.z / 3;
  const int c8 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c8 >= p.C) return;
  const int t0 = blockIdx.y * p.tokens_per_block;
  const int t1 = min(t0 + p.tokens_per_block, p.T);
  const int64_t C = p.C;
  const T* x = static_cast<const T*>(p.x[s]) + (int64_t)b * p.T * C + c8;
  T* y = static_cast<T*>(p.y[s]) + (int64_t)b * p.T * C + c8;
  const float* st_in = p.state_in ? p.state_in + ((int64_t)(b * 3 + s) * (W - 1)) * C + c8 : nullptr;

  float w[W][8];
#pragma unroll
  for (int ch = 0; ch < 8; ++ch)
#pragma unroll
    for (int j = 0; j < W; ++j) w[j][ch] = p.w[s][(int64_t)(c8 + ch) * W + j];

  // input at time tau (< t1): the sequence, or the state before token 0
  auto input_at = [&](int tau, float* v) {
    if (tau >= 0) {
      Vec8<T>::load(x + tau * C, v);
    } else if (st_in != nullptr) {
      const float* q = st_in + (int64_t)(tau + W - 1) * C;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = q[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
  };

  float win[W > 1 ? W - 1 : 1][8];  // inputs at t - (W - 1) .. t - 1
#pragma unroll
  for (int j = 0; j < W - 1; ++j) input_at(t0 - (W - 1) + j, win[j]);

  for (int t = t0; t < t1; t += kUnroll) {
    float cur[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) Vec8<T>::template load<true>(x + min(t + u, t1 - 1) * C, cur[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float out[8];
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        float acc = w[W - 1][ch] * cur[u][ch];  // the current token, then the older ones
#pragma unroll
        for (int j = W - 2; j >= 0; --j) acc = __builtin_fmaf(w[j][ch], win[j][ch], acc);
        out[ch] = acc * sigmoid_fast(acc);  // Swish
      }
      if (t + u < t1) Vec8<T>::store(y + (t + u) * C, out);
#pragma unroll
      for (int j = 0; j + 1 < W - 1; ++j)
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) win[j][ch] = win[j + 1][ch];
      if constexpr (W > 1) {
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) win[W - 2][ch] = cur[u][ch];
      }
    }
  }

  // the last block writes the new state: the W - 1 inputs before token T
  if (p.state_out != nullptr && t1 == p.T) {
    float* st_out = p.state_out + ((int64_t)(b * 3 + s) * (W - 1)) * C + c8;
    float v[W > 1 ? W - 1 : 1][8];
#pragma unroll
    for (int i = 0; i < W - 1; ++i) input_at(p.T - (W - 1) + i, v[i]);  // every read before any write
#pragma unroll
    for (int i = 0; i < W - 1; ++i)
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) st_out[(int64_t)i * C + ch] = v[i][ch];
  }
}

// beta = Sigmoid(logit), one element per thread
template <typename T>
__global__ __launch_bounds__(256) void kda_prep_beta_kernel(const T* logit, T* beta, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) beta[i] = Elem<T>::from_f32(sigmoid_fast(Elem<T>::to_f32(logit[i])));
}

// state_out = state_in (or zeros) when there are no tokens
__global__ __launch_bounds__(256) void kda_prep_state_copy_kernel(const float* in, float* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = in != nullptr ? in[i] : 0.0f;
}

template <typename T, int W>
void launch_conv_t(const InputPrepParams& p, hipStream_t s) {
  const dim3 grid((p.C / 8 + 255) / 256, (p.T + p.tokens_per_block - 1) / p.tokens_per_block, 3 * p.B);
  hipLaunchKernelGGL((kda_prep_conv_kernel<T, W>), grid, dim3(256), 0, s, p);
}

template <typename T>
void launch_prep_t(const InputPrepParams& p, hipStream_t s) {
  if (p.T == 0) {
    const int64_t n = (int64_t)p.B * 3 * (p.W - 1) * p.C;
    if (p.state_out != nullptr && p.state_out != p.state_in && n > 0)
      hipLaunchKernelGGL(kda_prep_state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p.state_in,
                         p.state_out, n);
    return;
  }
  switch (p.W) {
    case 1: launch_conv_t<T, 1>(p, s); break;
    case 2: launch_conv_t<T, 2>(p, s); break;
    case 3: launch_conv_t<T, 3>(p, s); break;
    default: launch_conv_t<T, 4>(p, s); break;
  }
  if (p.beta_logit != nullptr) {
    const int64_t n = (int64_t)p.B * p.T * p.H;
    hipLaunchKernelGGL((kda_prep_beta_kernel<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const T*>(p.beta_logit), static_cast<T*>(p.beta), n);
  }
}

}  // namespace

hipError_t launch_input_prep(const InputPrepParams& p, int in_f32, hipStream_t s) {
  if (in_f32)
    launch_prep_t<float>(p, s);
  else
    launch_prep_t<uint16_t>(p, s);
  return hipGetLastError();
}

}  // namespace kda
