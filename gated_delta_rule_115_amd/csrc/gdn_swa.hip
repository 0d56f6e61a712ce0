// Softmax decode step over sink tokens and a sliding window, gfx950.
// "The Key to Going Linear: Analysis-Driven Transformer Linearization",
// section 4 ("Adding Sliding Window Attention"): the exact path attends to
// the first s tokens and the w most recent ones,
//   y^swa_t = sum_{i in I} exp(q_t.k_i * sm) v_i / sum_{i in I} exp(q_t.k_i * sm),
// and the layer output adds this to the linear state's read-out.
//
// HBM-bound: every cached key and value of the (b, h) is streamed once.  One
// work-group per (b, h); a group of D/8 lanes owns one key at a time (8
// elements per lane, one 16-byte load for bf16), so a wave covers 64/(D/8)
// keys per step and each lane group keeps its own running max / sum /
// accumulator (online softmax, f32).  Groups are merged through LDS at the end.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <class TIn>
__device__ __forceinline__ void ld8(const TIn* p, float* f) {
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
__device__ __forceinline__ void copy8(TIn* dst, const TIn* src) {
  if constexpr (sizeof(TIn) == 2) {
    *reinterpret_cast<bf16x8*>(dst) = *reinterpret_cast<const bf16x8*>(src);
  } else {
    *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(src);
    *reinterpret_cast<f32x4*>(dst + 4) = *reinterpret_cast<const f32x4*>(src + 4);
  }
}

template <class TIn, class TOut, int D>
__global__ __launch_bounds__(256) void swa_sink_decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k_new,
    const TIn* __restrict__ v_new, TIn* __restrict__ k_cache,
    TIn* __restrict__ v_cache, const int* __restrict__ n_tokens, int H,
    int n_sink, int window, float sm_scale, int accumulate, TOut* __restrict__ out) {
  constexpr int LPK = D / 8;             // lanes per key
  constexpr int KPW = kWave / LPK;       // keys per wave per step
  constexpr int NG = 4 * KPW;            // lane groups per work-group
  constexpr int UNR = 4;                 // keys per lane group per step

  __shared__ float gm[NG], gs[NG];
  __shared__ float gacc[NG][D + 4];

  const int bh = blockIdx.x;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = lane_id();
  const int grp = wave * KPW + l / LPK;  // lane group id
  const int sub = l % LPK;               // this lane's 8-element piece
  const int nslot = n_sink + window;
  const size_t cbase = (size_t)bh * nslot * D;

  const int t = n_tokens[b];  // tokens seen, current at position t-1
  const int n_s = max(0, min(n_sink, t));
  const int n_w = max(0, min(window, t - n_sink));
  const int n_valid = n_s + n_w;
  int cur = -1;  // slot of the current token
  if (t >= 1) cur = (t - 1 < n_sink) ? (t - 1) : n_sink + (t - 1 - n_sink) % window;
  const bool have_new = (k_new != nullptr);

  // Store the current token into its slot (overwrites the evicted token).
  if (have_new && cur >= 0 && wave == 0 && l < LPK) {
    copy8(k_cache + cbase + (size_t)cur * D + l * 8, k_new + (size_t)bh * D + l * 8);
    copy8(v_cache + cbase + (size_t)cur * D + l * 8, v_new + (size_t)bh * D + l * 8);
  }

  float qf[8];
  ld8(q + (size_t)bh * D + sub * 8, qf);
#pragma unroll
  for (int e = 0; e < 8; ++e) qf[e] *= sm_scale;

  float m = -INFINITY, s = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;

  // Valid slots are [0, n_s) and [n_sink, n_sink + n_w): enumerate as j in
  // [0, n_valid) -> slot(j).
  for (int j0 = grp * UNR; j0 < n_valid; j0 += NG * UNR) {
    float kf[UNR][8], vf[UNR][8];
    bool ok[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = j0 + u;
      ok[u] = j < n_valid;
      const int slot = (j < n_s) ? j : n_sink + (j - n_s);
      const TIn* kp;
      const TIn* vp;
      if (have_new && slot == cur) {
        kp = k_new + (size_t)bh * D;
        vp = v_new + (size_t)bh * D;
      } else {
        kp = k_cache + cbase + (size_t)slot * D;
        vp = v_cache + cbase + (size_t)slot * D;
      }
      if (ok[u]) {
        ld8(kp + sub * 8, kf[u]);
        ld8(vp + sub * 8, vf[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[u][e] = vf[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float z = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) z += qf[e] * kf[u][e];
#pragma unroll
      for (int off = 1; off < LPK; off <<= 1) z += __shfl_xor(z, off);
      if (ok[u]) {
        const float mn = fmaxf(m, z);
        const float corr = __expf(m - mn);
        const float p = __expf(z - mn);
        s = s * corr + p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] * corr + p * vf[u][e];
        m = mn;
      }
    }
  }

  if (sub == 0) {
    gm[grp] = m;
    gs[grp] = s;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) gacc[grp][sub * 8 + e] = acc[e];
  __syncthreads();

  if (tid < D) {
    float M = -INFINITY;
    for (int g = 0; g < NG; ++g) M = fmaxf(M, gm[g]);
    float den = 0.f, num = 0.f;
    for (int g = 0; g < NG; ++g) {
      if (gm[g] == -INFINITY) continue;
      const float w = __expf(gm[g] - M);
      den += w * gs[g];
      num += w * gacc[g][tid];
    }
    float yv = (den > 0.f) ? num / den : 0.f;
    TOut* o = out + (size_t)bh * D + tid;
    if (accumulate) yv += to_f32(*o);
    *o = from_f32<TOut>(yv);
  }
}

template <class TIn, class TOut, int D>
static hipError_t launch_swa_t(const SwaArgs& p) {
  hipLaunchKernelGGL((swa_sink_decode_kernel<TIn, TOut, D>), dim3(p.B * p.H), dim3(256), 0,
                     (hipStream_t)p.stream, (const TIn*)p.q, (const TIn*)p.k_new,
                     (const TIn*)p.v_new, (TIn*)p.k_cache, (TIn*)p.v_cache, p.n_tokens,
                     p.H, p.n_sink, p.window, p.softmax_scale, p.accumulate,
                     (TOut*)p.out);
  return hipGetLastError();
}

template <class TIn, class TOut>
static hipError_t launch_swa_d(const SwaArgs& p) {
  switch (p.D) {
    case 64: return launch_swa_t<TIn, TOut, 64>(p);
    case 128: return launch_swa_t<TIn, TOut, 128>(p);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_swa(const SwaArgs& p) {
  if (p.B * p.H == 0) return hipSuccess;
  if (!p.bf16) return launch_swa_d<float, float>(p);
  return p.out_bf16 ? launch_swa_d<bf16, bf16>(p) : launch_swa_d<bf16, float>(p);
}

}  // namespace gdn
