// Causal depthwise short convolution + SiLU (+ per-head L2 normalisation),
// gfx950.  "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 4 ("Adapting Q/K/V": short convolutions on the q,
// k, v projections); the normalisation is the key normalisation
// k / (||k||_2 + eps) of appendix B.1.
//
//   y_t[c] = SiLU( sum_{j<K} taps[c][j] * x_{t-K+1+j}[c] ),   x_{<0} = 0
//
// Elementwise stencil, HBM-bound.  One thread owns 8 consecutive channels and
// walks a run of consecutive tokens, keeping the last K-1 input rows in
// registers, so every input element is read from memory once per run (plus a
// K-1 row halo) and every output is written once with 16-byte accesses.  The
// run is taken in blocks of rows whose loads are all issued before any is
// used, and the next block is loaded while the current one is computed.  L2 groups (a head's channels) are
// consecutive lanes of one wave, reduced with cross-lane shuffles.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// Outputs are written with non-temporal stores: each is written once and the
// stream is larger than the caches.
template <class TIn>
__device__ __forceinline__ void store8(TIn* p, const float* f) {
  if constexpr (sizeof(TIn) == 2) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (bf16)f[e];
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x), reinterpret_cast<u32x4*>(p));
  } else {
    __builtin_nontemporal_store(f32x4{f[0], f[1], f[2], f[3]}, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(f32x4{f[4], f[5], f[6], f[7]}, reinterpret_cast<f32x4*>(p + 4));
  }
}

// Raw 8-channel piece as loaded (bf16: one 16-byte load; f32: two).
template <class TIn>
struct Raw8 {
  bf16x8 v;
};
template <>
struct Raw8<float> {
  f32x4 a, b;
};
template <class TIn>
__device__ __forceinline__ Raw8<TIn> load_raw8(const TIn* p) {
  Raw8<TIn> r;
  if constexpr (sizeof(TIn) == 2) {
    r.v = *reinterpret_cast<const bf16x8*>(p);
  } else {
    r.a = *reinterpret_cast<const f32x4*>(p);
    r.b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  return r;
}
template <class TIn>
__device__ __forceinline__ float raw8_at(const Raw8<TIn>& r, int e) {
  if constexpr (sizeof(TIn) == 2) {
    return (float)r.v[e];
  } else {
    return e < 4 ? r.a[e] : r.b[e - 4];
  }
}

constexpr int kConvThreads = 128;
constexpr int kConvRun = 128;  // tokens per thread
constexpr int kConvBlk = 8;    // tokens whose loads are in flight together

template <class TIn, class TOut, int K>
__global__ __launch_bounds__(kConvThreads) void short_conv_silu_kernel(
    const TIn* __restrict__ x, const float* __restrict__ taps,
    TOut* __restrict__ y, int T, int Ch, int group, float eps) {
  const int nvec = Ch / 8;
  const int vi = blockIdx.x * kConvThreads + threadIdx.x;  // channel vector index
  const bool active = vi < nvec;
  const int b = blockIdx.z;
  const int tb = blockIdx.y * kConvRun;
  const int te = min(T, tb + kConvRun);
  const int c0 = (active ? vi : nvec - 1) * 8;
  const TIn* xb = x + (size_t)b * T * Ch + c0;
  TOut* yb = y + (size_t)b * T * Ch + c0;

  // Taps and history loads are unconditional (an inactive thread reads the
  // last channel vector; rows before the sequence read row 0 and are zeroed
  // after the load), so they are all in flight together.
  float w[8][K];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int j = 0; j < K; ++j) w[e][j] = taps[(size_t)(c0 + e) * K + j];

  // History rows x_{t-K+1} .. x_{t-1} (oldest first).
  float hist[K > 1 ? K - 1 : 1][8];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int ts = tb - (K - 1) + j;
    const Raw8<TIn> r = load_raw8(xb + (size_t)max(ts, 0) * Ch);
#pragma unroll
    for (int e = 0; e < 8; ++e) hist[j][e] = ts >= 0 ? raw8_at(r, e) : 0.f;
  }

  const int gl = group / 8;  // lanes per L2 group (0 = no normalisation)
  // Rows of block t0 .. t0 + kConvBlk - 1.  Past the run the last row is
  // loaded again (its results are not stored), so every block issues the
  // same loads without branches; an inactive thread reads channel 0.
  auto fetch = [&](int t0, Raw8<TIn>* rows) {
#pragma unroll
    for (int u = 0; u < kConvBlk; ++u) rows[u] = load_raw8(xb + (size_t)min(t0 + u, te - 1) * Ch);
  };
  auto consume = [&](int t0, const Raw8<TIn>* rows) {
#pragma unroll
    for (int u = 0; u < kConvBlk; ++u) {
      const int t = t0 + u;
      float cur[8], o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cur[e] = raw8_at(rows[u], e);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float a = w[e][K - 1] * cur[e];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) a += w[e][j] * hist[j][e];
        o[e] = a * __builtin_amdgcn_rcpf(1.f + __expf(-a));  // hardware reciprocal
        ss += o[e] * o[e];
      }
      if (gl > 0) {
        for (int m = 1; m < gl; m <<= 1) ss += __shfl_xor(ss, m);
        const float inv = __builtin_amdgcn_rcpf(sqrtf(ss) + eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= inv;
      }
      if (active && t < te) store8(yb + (size_t)t * Ch, o);
#pragma unroll
      for (int j = 0; j + 1 < K - 1; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) hist[j][e] = hist[j + 1][e];
      if (K > 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) hist[K > 1 ? K - 2 : 0][e] = cur[e];
    }
  };
  // Two blocks in flight: block b + 1 is loaded before block b is consumed.
  Raw8<TIn> ra[kConvBlk], rb[kConvBlk];
  fetch(tb, ra);
  for (int t0 = tb; t0 < te; t0 += 2 * kConvBlk) {
    const int t1 = t0 + kConvBlk;
    if (t1 < te) fetch(t1, rb);
    consume(t0, ra);
    if (t1 < te) {
      if (t1 + kConvBlk < te) fetch(t1 + kConvBlk, ra);
      consume(t1, rb);
    }
  }
}

template <class TIn, class TOut, int K>
static hipError_t launch_conv_t(const ConvArgs& p) {
  const int nvec = p.Ch / 8;
  dim3 grid((nvec + kConvThreads - 1) / kConvThreads, (p.T + kConvRun - 1) / kConvRun, p.B);
  hipLaunchKernelGGL((short_conv_silu_kernel<TIn, TOut, K>), grid, dim3(kConvThreads), 0,
                     (hipStream_t)p.stream, (const TIn*)p.x, p.taps, (TOut*)p.y, p.T,
                     p.Ch, p.group, p.eps);
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

// One decode step: the same convolution at one new token per sequence, from
// the K - 1 previous inputs of each channel kept in `state` [B][K-1][Ch]
// (oldest row first), which is then shifted by one row with the new token
// appended.  A thread owns 8 channels of one sequence: it reads the token and
// its history rows, writes y and the shifted history (every thread reads its
// own channels before writing them, so the update is in place).  The
// work-groups of a sequence are consecutive (no per-thread division), and
// every load is unconditional (lanes past the last channel vector read the
// last one and store nothing), so all of a thread's loads are in flight
// together.  L2 groups are consecutive lanes of one wave (a group's channels
// are consecutive, and a work-group's 128 vectors start at a multiple of 128).
template <class TIn, class TOut, int K>
__global__ __launch_bounds__(kConvThreads) void short_conv_step_kernel(
    const TIn* __restrict__ x, const float* __restrict__ taps, TIn* __restrict__ state,
    TOut* __restrict__ y, int B, int Ch, int group, float eps) {
  const int nvec = Ch / 8;
  const int nblk = (nvec + kConvThreads - 1) / kConvThreads;  // work-groups per sequence
  const int b = blockIdx.x / nblk;
  const int vi = (blockIdx.x - b * nblk) * kConvThreads + threadIdx.x;
  const bool active = vi < nvec;
  const int c0 = min(vi, nvec - 1) * 8;
  float w[8][K];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int j = 0; j < K; ++j) w[e][j] = taps[(size_t)(c0 + e) * K + j];
  Raw8<TIn> rows[K];  // history rows 0 .. K - 2, then the new token
  TIn* sb = state + (size_t)b * (K - 1) * Ch + c0;
#pragma unroll
  for (int j = 0; j < K; ++j)
    rows[j] = load_raw8(j < K - 1 ? sb + (size_t)j * Ch : x + (size_t)b * Ch + c0);
  float o[8], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) a += w[e][j] * raw8_at(rows[j], e);
    o[e] = a * __builtin_amdgcn_rcpf(1.f + __expf(-a));
    ss += o[e] * o[e];
  }
  const int gl = group / 8;
  if (gl > 0) {
    if (!active) ss = 0.f;
    for (int m = 1; m < gl; m <<= 1) ss += __shfl_xor(ss, m);
    const float inv = __builtin_amdgcn_rcpf(sqrtf(ss) + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv;
  }
  if (!active) return;
  store8(y + (size_t)b * Ch + c0, o);
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = raw8_at(rows[j + 1], e);
    store8(sb + (size_t)j * Ch, f);
  }
}

template <class TIn, class TOut, int K>
static hipError_t launch_conv_step_t(const ConvArgs& p, void* state) {
  const long long n = (long long)p.B * ((p.Ch / 8 + kConvThreads - 1) / kConvThreads);
  hipLaunchKernelGGL((short_conv_step_kernel<TIn, TOut, K>), dim3((unsigned)n), dim3(kConvThreads), 0,
                     (hipStream_t)p.stream, (const TIn*)p.x, p.taps, (TIn*)state, (TOut*)p.y, p.B,
                     p.Ch, p.group, p.eps);
  return hipGetLastError();
}

template <class TIn, class TOut>
static hipError_t launch_conv_step_k(const ConvArgs& p, void* state) {
  switch (p.K) {
    case 1: return launch_conv_step_t<TIn, TOut, 1>(p, state);
    case 2: return launch_conv_step_t<TIn, TOut, 2>(p, state);
    case 3: return launch_conv_step_t<TIn, TOut, 3>(p, state);
    case 4: return launch_conv_step_t<TIn, TOut, 4>(p, state);
    case 5: return launch_conv_step_t<TIn, TOut, 5>(p, state);
    case 6: return launch_conv_step_t<TIn, TOut, 6>(p, state);
    case 7: return launch_conv_step_t<TIn, TOut, 7>(p, state);
    case 8: return launch_conv_step_t<TIn, TOut, 8>(p, state);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv_step(const ConvArgs& p, void* state) {
  if (p.B == 0) return hipSuccess;
  if (!p.bf16) return launch_conv_step_k<float, float>(p, state);
  return p.out_bf16 ? launch_conv_step_k<bf16, bf16>(p, state)
                    : launch_conv_step_k<bf16, float>(p, state);
}

hipError_t launch_conv(const ConvArgs& p) {
  if ((long)p.B * p.T == 0) return hipSuccess;
  if (!p.bf16) return launch_conv_k<float, float>(p);
  return p.out_bf16 ? launch_conv_k<bf16, bf16>(p) : launch_conv_k<bf16, float>(p);
}

}  // namespace gdn
