// Causal depthwise short convolution + SiLU (+ per-head L2 normalisation),
// gfx950.  "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 4 ("Adapting Q/K/V": short convolutions on the q,
// k, v projections); the normalisation is the key normalisation
// k / (||k||_2 + eps) of appendix B.1.
//
//   y_t[c] = SiLU( sum_{j<K} taps[c][j] * x_{t-K+1+j}[c] ),   x_{<0} = 0
//
// Elementwise stencil, HBM-bound.  One thread owns 8 consecutive channels and
// walks TT consecutive tokens, keeping the last K-1 input rows in registers,
// so every input element is read from memory once per token run (plus a
// K-1 row halo) and every output is written once with 16-byte accesses.
// L2 groups (a head's channels) are consecutive lanes of one wave, reduced
// with cross-lane shuffles.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <class TIn>
__device__ __forceinline__ void load8(const TIn* p, float* f) {
  if constexpr (sizeof(TIn) == 2) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (float)x[e];
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = a[e];
      f[4 + e] = b[e];
    }
  }
}

template <class TIn>
__device__ __forceinline__ void store8(TIn* p, const float* f) {
  if constexpr (sizeof(TIn) == 2) {
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (bf16)f[e];
    *reinterpret_cast<bf16x8*>(p) = x;
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
  }
}

template <class TIn, class TOut, int K>
__global__ __launch_bounds__(256) void short_conv_silu_kernel(
    const TIn* __restrict__ x, const float* __restrict__ taps,
    TOut* __restrict__ y, int T, int Ch, int group, float eps, int TT) {
  const int nvec = Ch / 8;
  const int vi = blockIdx.x * 256 + threadIdx.x;  // channel vector index
  const bool active = vi < nvec;
  const int b = blockIdx.z;
  const int tb = blockIdx.y * TT;
  const int te = min(T, tb + TT);
  const int c0 = (active ? vi : 0) * 8;

  float w[8][K];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int j = 0; j < K; ++j) w[e][j] = active ? taps[(size_t)(c0 + e) * K + j] : 0.f;

  // History rows x_{t-K+1} .. x_{t-1} (oldest first).
  float hist[K > 1 ? K - 1 : 1][8];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int ts = tb - (K - 1) + j;
    if (active && ts >= 0)
      load8(x + ((size_t)b * T + ts) * Ch + c0, hist[j]);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) hist[j][e] = 0.f;
  }

  const int gl = group / 8;  // lanes per L2 group (0 = no normalisation)
  for (int t = tb; t < te; ++t) {
    float cur[8], o[8];
    if (active)
      load8(x + ((size_t)b * T + t) * Ch + c0, cur);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) cur[e] = 0.f;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = w[e][K - 1] * cur[e];
#pragma unroll
      for (int j = 0; j < K - 1; ++j) a += w[e][j] * hist[j][e];
      o[e] = a / (1.f + __expf(-a));
      ss += o[e] * o[e];
    }
    if (gl > 0) {
      for (int m = 1; m < gl; m <<= 1) ss += __shfl_xor(ss, m);
      const float inv = 1.f / (sqrtf(ss) + eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= inv;
    }
    if (active) store8(y + ((size_t)b * T + t) * Ch + c0, o);
#pragma unroll
    for (int j = 0; j + 1 < K - 1; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) hist[j][e] = hist[j + 1][e];
    if (K > 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) hist[K > 1 ? K - 2 : 0][e] = cur[e];
  }
}

template <class TIn, class TOut, int K>
static hipError_t launch_conv_t(const ConvArgs& p) {
  const int TT = 64;
  const int nvec = p.Ch / 8;
  dim3 grid((nvec + 255) / 256, (p.T + TT - 1) / TT, p.B);
  hipLaunchKernelGGL((short_conv_silu_kernel<TIn, TOut, K>), grid, dim3(256), 0,
                     (hipStream_t)p.stream, (const TIn*)p.x, p.taps, (TOut*)p.y, p.T,
                     p.Ch, p.group, p.eps, TT);
  return hipGetLastError();
}

template <class TIn, class TOut>
static hipError_t launch_conv_k(const ConvArgs& p) {
  switch (p.K) {
    case 1: return launch_conv_t<TIn, TOut, 1>(p);
    case 2: return launch_conv_t<TIn, TOut, 2>(p);
    case 3: return launch_conv_t<TIn, TOut, 3>(p);
    case 4: return launch_conv_t<TIn, TOut, 4>(p);
    case 5: return launch_conv_t<TIn, TOut, 5>(p);
    case 6: return launch_conv_t<TIn, TOut, 6>(p);
    case 7: return launch_conv_t<TIn, TOut, 7>(p);
    case 8: return launch_conv_t<TIn, TOut, 8>(p);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv(const ConvArgs& p) {
  if ((long)p.B * p.T == 0) return hipSuccess;
  if (!p.bf16) return launch_conv_k<float, float>(p);
  return p.out_bf16 ? launch_conv_k<bf16, bf16>(p) : launch_conv_k<bf16, float>(p);
}

}  // namespace gdn
