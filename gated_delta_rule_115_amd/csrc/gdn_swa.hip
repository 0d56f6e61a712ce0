// Softmax decode step over sink tokens and a sliding window, gfx950.
// "The Key to Going Linear: Analysis-Driven Transformer Linearization",
// section 4 ("Adding Sliding Window Attention"): the exact path attends to
// the first s tokens and the w most recent ones,
//   y^swa_t = sum_{i in I} exp(q_t.k_i * sm) v_i / sum_{i in I} exp(q_t.k_i * sm),
// and the layer output adds this to the linear state's read-out.
//
// HBM-bound: every cached key and value of the (b, h) is streamed once.  One
// work-group per (b, h); a group of D/8 lanes owns one key at a time (8
// elements per lane, one 16-byte load for bf16).  Each lane group takes UNR
// keys per step, the groups of a wave reading consecutive keys, and NBUF steps
// of loads are in flight (a software pipeline whose buffers are registers).
// Each group keeps its own running max / sum / accumulator (online softmax,
// f32, one rescale per step); groups are merged through LDS at the end.
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
// Cache rows are streamed with non-temporal loads: each is read once per
// step, and the scan is several times larger than the caches.
template <class TIn>
__device__ __forceinline__ Piece<TIn> load_piece(const TIn* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  Piece<TIn> r;
  if constexpr (sizeof(TIn) == 2) {
    r.v = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
  } else {
    r.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    r.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
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

// Sum over the LPK lanes of a row group (LPK = 8 or 16, groups aligned to
// 8 or 16 lanes) with DPP row permutations: swap neighbours, swap pairs,
// mirror within 8 lanes, mirror within 16 lanes.  Every lane of the group
// ends with the total.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int LPK>
__device__ __forceinline__ float group_sum(float d) {
  static_assert(LPK == 8 || LPK == 16, "lane groups of 8 or 16");
  d += dpp_f<0xB1>(d);   // quad_perm [1, 0, 3, 2]
  d += dpp_f<0x4E>(d);   // quad_perm [2, 3, 0, 1]
  d += dpp_f<0x141>(d);  // row_half_mirror
  if constexpr (LPK == 16) d += dpp_f<0x140>(d);  // row_mirror
  return d;
}

// NT threads per work-group; each lane group takes UNR keys per step and
// NBUF steps are in flight (the loads of step s + NBUF - 1 are issued before
// step s is consumed).  Past the last valid key the loads repeat that key
// (same cache lines, no extra HBM traffic) and its weight is zero, so every
// step issues the same loads without branches and the waits are fixed counts.
template <class TIn, class TOut, int D, int NT, int UNR, int NBUF>
__global__ __launch_bounds__(NT) void swa_sink_decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k_new,
    const TIn* __restrict__ v_new, TIn* __restrict__ k_cache,
    TIn* __restrict__ v_cache, const int* __restrict__ n_tokens, int H,
    int n_sink, int window, float sm_scale, int accumulate, TOut* __restrict__ out) {
  constexpr int LPK = D / 8;             // lanes per key
  constexpr int KPW = kWave / LPK;       // keys per wave per load
  constexpr int NG = (NT / kWave) * KPW; // lane groups per work-group
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
  Piece<TIn> kr[NBUF][UNR], vr[NBUF][UNR];
  auto fetch = [&](int st, Piece<TIn>* kk, Piece<TIn>* vv) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = min(st * STEP + u * NG + grp, n_valid - 1);
      const int slot = (j < n_s) ? j : n_sink + (j - n_s);
      const bool fresh = have_new && slot == cur;
      const TIn* kp = fresh ? k_new + (size_t)bh * D : k_cache + cbase + (size_t)slot * D;
      const TIn* vp = fresh ? v_new + (size_t)bh * D : v_cache + cbase + (size_t)slot * D;
      kk[u] = load_piece(kp + sub * 8);
      vv[u] = load_piece(vp + sub * 8);
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
      d = group_sum<LPK>(d);
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

  // Software pipeline over steps, NBUF deep; buffer indices are compile-time.
  const int nsteps = (n_valid + STEP - 1) / STEP;
#pragma unroll
  for (int bb = 0; bb + 1 < NBUF; ++bb)
    if (bb < nsteps) fetch(bb, kr[bb], vr[bb]);
  for (int st = 0; st < nsteps; st += NBUF) {
#pragma unroll
    for (int bb = 0; bb < NBUF; ++bb) {
      const int sc = st + bb;
      if (sc < nsteps) {
        if (sc + NBUF - 1 < nsteps)
          fetch(sc + NBUF - 1, kr[(bb + NBUF - 1) % NBUF], vr[(bb + NBUF - 1) % NBUF]);
        consume(sc, kr[bb], vr[bb]);
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

// Work-group shape per element type: bf16 keys are one 16-byte load per lane.
template <class TIn>
struct SwaShape {
  static constexpr int NT = 512, UNR = 4, NBUF = 2;
};
template <>
struct SwaShape<float> {
  static constexpr int NT = 256, UNR = 4, NBUF = 2;
};

template <class TIn, class TOut, int D>
static hipError_t launch_swa_t(const SwaArgs& p) {
  typedef SwaShape<TIn> Sh;
  hipLaunchKernelGGL((swa_sink_decode_kernel<TIn, TOut, D, Sh::NT, Sh::UNR, Sh::NBUF>),
                     dim3(p.B * p.H), dim3(Sh::NT), 0,
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
