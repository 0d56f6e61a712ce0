// Softmax decode step over sink tokens and a sliding window, gfx950.
// "The Key to Going Linear: Analysis-Driven Transformer Linearization",
// section 4 ("Adding Sliding Window Attention"): the exact path attends to
// the first s tokens and the w most recent ones,
//   y^swa_t = sum_{i in I} exp(q_t.k_i * sm) v_i / sum_{i in I} exp(q_t.k_i * sm),
// and the layer output adds this to the linear state's read-out.
//
// HBM-bound: every cached key and value of the (b, h) is streamed once.  One
// work-group per (b, h); a group of D/8 lanes owns one key at a time (8
// elements per lane, one 16-byte load for bf16).  Each lane group takes 8 keys
// per step, the groups of a wave reading consecutive keys, and the next step's
// keys and values are loaded before the current step is consumed.  Each group
// keeps its own running max / sum / accumulator (online softmax, f32, one
// rescale per step); groups are merged through LDS at the end.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// Raw 8-element piece as loaded (bf16: one 16-byte load; f32: two).
template <class TIn>
struct Piece {
  bf16x8 v;
};
template <>
struct Piece<float> {
  f32x4 a, b;
};
template <class TIn>
__device__ __forceinline__ Piece<TIn> load_piece(const TIn* p) {
  Piece<TIn> r;
  if constexpr (sizeof(TIn) == 2) {
    r.v = *reinterpret_cast<const bf16x8*>(p);
  } else {
    r.a = *reinterpret_cast<const f32x4*>(p);
    r.b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  return r;
}
template <class TIn>
__device__ __forceinline__ Piece<TIn> zero_piece() {
  Piece<TIn> r;
  if constexpr (sizeof(TIn) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r.v[e] = (bf16)0.f;
  } else {
    r.a = zero4();
    r.b = zero4();
  }
  return r;
}
template <class TIn>
__device__ __forceinline__ float piece_at(const Piece<TIn>& r, int e) {
  if constexpr (sizeof(TIn) == 2) {
    return (float)r.v[e];
  } else {
    return e < 4 ? r.a[e] : r.b[e - 4];
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
  constexpr int KPW = kWave / LPK;       // keys per wave per load
  constexpr int NG = 4 * KPW;            // lane groups per work-group
  constexpr int UNR = 8;                 // keys per lane group per step
  constexpr int STEP = NG * UNR;         // keys per step

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
  {
    const Piece<TIn> qp = load_piece(q + (size_t)bh * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = piece_at(qp, e) * sm_scale;
  }

  // Valid slots are [0, n_s) and [n_sink, n_sink + n_w): position j in
  // [0, n_valid) -> slot(j).  Step s, piece u of group g: j = s STEP + u NG + g,
  // so the groups of a wave read consecutive keys.
  Piece<TIn> kr[2][UNR], vr[2][UNR];
  auto fetch = [&](int st, Piece<TIn>* kk, Piece<TIn>* vv) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = st * STEP + u * NG + grp;
      if (j < n_valid) {
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
        kk[u] = load_piece(kp + sub * 8);
        vv[u] = load_piece(vp + sub * 8);
      } else {
        kk[u] = zero_piece<TIn>();  // weight 0 below; must not hold NaN
        vv[u] = zero_piece<TIn>();
      }
    }
  };

  float m = -INFINITY, s = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  auto consume = [&](int st, const Piece<TIn>* kk, const Piece<TIn>* vv) {
    float z[UNR];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d += qf[e] * piece_at(kk[u], e);
#pragma unroll
      for (int off = 1; off < LPK; off <<= 1) d += __shfl_xor(d, off);
      const bool ok = st * STEP + u * NG + grp < n_valid;
      z[u] = ok ? d : -INFINITY;
      mx = fmaxf(mx, z[u]);
    }
    if (mx == -INFINITY) return;  // no valid key for this group in this step
    const float mn = fmaxf(m, mx);
    const float corr = __expf(m - mn);
    s *= corr;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= corr;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const float pr = __expf(z[u] - mn);  // 0 for the invalid pieces
      s += pr;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += pr * piece_at(vv[u], e);
    }
    m = mn;
  };

  // Two steps in flight: step s + 1 is loaded before step s is consumed.
  const int nsteps = (n_valid + STEP - 1) / STEP;
  if (nsteps > 0) fetch(0, kr[0], vr[0]);
  for (int st = 0; st < nsteps; st += 2) {
    if (st + 1 < nsteps) fetch(st + 1, kr[1], vr[1]);
    consume(st, kr[0], vr[0]);
    if (st + 1 < nsteps) {
      if (st + 2 < nsteps) fetch(st + 2, kr[0], vr[0]);
      consume(st + 1, kr[1], vr[1]);
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
