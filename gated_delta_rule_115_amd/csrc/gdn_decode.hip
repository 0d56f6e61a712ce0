// Single-token GDN decode step for a batch of sequences, gfx950.
//
// "The Key to Going Linear: Analysis-Driven Transformer Linearization",
// section 3.1.2 (recurrent form), one token per (b, h):
//   S' = alpha (I - beta k k^T) S + beta k v^T,   out = scale * S'^T q.
// Rewritten so the state is touched in ONE pass (read once, written once):
//   u   = beta (v - alpha S^T k)                 [Dv]
//   out = scale (alpha S^T q + (k . q) u)        [Dv]
//   S'  = alpha S + k u^T
// (expand S' and substitute; it is the same update exactly).
//
// The step is HBM-bound: 8*Dk*Dv bytes of f32 state per (b, h) against
// ~4*Dk*Dv flops.  One work-group owns one (b, h); thread (rg, cg) holds
// rows rg, rg+RG, ... and the float4 column group cg of S in registers, so every state load/store is a 16-byte coalesced access and all
// of a thread's loads are in flight before the first reduction.  The new
// state is written with non-temporal stores: it is far larger than the caches
// and is not read again within the step, and keeping its lines out of the
// caches leaves no write-back to compete with the reads of the kernel that
// follows (the softmax path's cache scan).  Measured on the hybrid decode
// step, this beats both ordinary stores and non-temporal loads as well.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// MODE 0: scalar gate alpha [B, H].
// MODE 1: channel-wise gate, alpha is [B, H, DK] and row r of S is scaled by
// alpha[r] before the step (G_t = diag(alpha_t) applied first, as in the
// page's update); the step then runs with a = 1.
// MODE 2: gated linear attention with a key-dependent gate (section 3.2.2):
// row r of S is scaled by alpha[r] (1 - beta k[r]^2), there is no erase and
// the write is k v^T, so u = v.
// Threads per work-group: DK * DV / 32 (16 state values per thread), at
// least 64 and DV (one thread per column in the reduction), at most 512.
// At 128 x 128, 512 threads (8 rows of one float4 column group each) ran the
// B256 H32 step 3-4 % faster than 256 threads with 16 rows.
template <int DK, int DV>
constexpr int decode_threads() {
  constexpr int n = DK * DV / 32 < 64 ? 64 : (DK * DV / 32 > 512 ? 512 : DK * DV / 32);
  return n < DV ? DV : n;
}

template <class TIn, class TOut, int DK, int DV, int MODE>
__global__ __launch_bounds__((decode_threads<DK, DV>())) void decode_step_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* state_in, float* state_out,
    TOut* __restrict__ out, float scale) {
  constexpr int NT = decode_threads<DK, DV>();
  constexpr int CG = DV / 4;            // float4 column groups
  constexpr int RG = NT / CG;           // row groups
  constexpr int RPT = (DK + RG - 1) / RG;  // rows per thread
  static_assert(NT % CG == 0, "DV/4 must divide the thread count");

  __shared__ float ks[DK], qs[DK], vs[DV];
  __shared__ float red_k[RG][DV + 4], red_q[RG][DV + 4];
  __shared__ float red_kq[RG];
  __shared__ float us[DV];

  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const size_t sbase = (size_t)bh * DK * DV;

  // State rows of this thread, all loads issued up front.
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + i * RG;
    if (r < DK)
      s[i] = *reinterpret_cast<const f32x4*>(state_in + sbase + (size_t)r * DV + cg * 4);
    else
      s[i] = zero4();
  }

  for (int i = tid; i < DK; i += NT) {
    ks[i] = to_f32(k[(size_t)bh * DK + i]);
    qs[i] = to_f32(q[(size_t)bh * DK + i]);
  }
  for (int i = tid; i < DV; i += NT) vs[i] = to_f32(v[(size_t)bh * DV + i]);
  const float a = MODE == 0 ? alpha[bh] : 1.f;
  const float b = beta[bh];
  if constexpr (MODE == 1) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + i * RG;
      if (r < DK) s[i] *= alpha[(size_t)bh * DK + r];
    }
  }
  __syncthreads();
  if constexpr (MODE == 2) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + i * RG;
      if (r < DK) s[i] *= alpha[(size_t)bh * DK + r] * (1.f - b * ks[r] * ks[r]);
    }
  }

  // Partial S^T k and S^T q over this thread's rows; k.q from column group 0.
  float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
  float pkq = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + i * RG;
    if (r < DK) {
      const float kr = ks[r], qr = qs[r];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pk[c] += s[i][c] * kr;
        pq[c] += s[i][c] * qr;
      }
      if (cg == 0) pkq += kr * qr;
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    red_k[rg][cg * 4 + c] = pk[c];
    red_q[rg][cg * 4 + c] = pq[c];
  }
  if (cg == 0) red_kq[rg] = pkq;
  __syncthreads();

  if (tid < DV) {
    float sk = 0.f, sq = 0.f, kq = 0.f;
    for (int g = 0; g < RG; ++g) {
      sk += red_k[g][tid];
      sq += red_q[g][tid];
      kq += red_kq[g];
    }
    const float u = MODE == 2 ? vs[tid] : b * (vs[tid] - a * sk);
    us[tid] = u;
    out[(size_t)bh * DV + tid] = from_f32<TOut>(scale * (a * sq + kq * u));
  }
  __syncthreads();

  const f32x4 u4 = *reinterpret_cast<const f32x4*>(&us[cg * 4]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + i * RG;
    if (r < DK) {
      const float kr = ks[r];
      f32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = a * s[i][c] + kr * u4[c];
      __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(state_out + sbase + (size_t)r * DV + cg * 4));
    }
  }
}

template <class TIn, class TOut, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& p) {
  if (p.chgate && p.kgla)
    hipLaunchKernelGGL((decode_step_kernel<TIn, TOut, DK, DV, 2>), dim3(p.B * p.H), dim3(decode_threads<DK, DV>()),
                       0, (hipStream_t)p.stream, (const TIn*)p.q, (const TIn*)p.k,
                       (const TIn*)p.v, p.alpha, p.beta, p.state_in, p.state_out,
                       (TOut*)p.out, p.scale);
  else if (p.chgate)
    hipLaunchKernelGGL((decode_step_kernel<TIn, TOut, DK, DV, 1>), dim3(p.B * p.H), dim3(decode_threads<DK, DV>()),
                       0, (hipStream_t)p.stream, (const TIn*)p.q, (const TIn*)p.k,
                       (const TIn*)p.v, p.alpha, p.beta, p.state_in, p.state_out,
                       (TOut*)p.out, p.scale);
  else
    hipLaunchKernelGGL((decode_step_kernel<TIn, TOut, DK, DV, 0>), dim3(p.B * p.H), dim3(decode_threads<DK, DV>()),
                       0, (hipStream_t)p.stream, (const TIn*)p.q, (const TIn*)p.k,
                       (const TIn*)p.v, p.alpha, p.beta, p.state_in, p.state_out,
                       (TOut*)p.out, p.scale);
  return hipGetLastError();
}

template <class TIn, class TOut, int DK>
static hipError_t launch_decode_dv(const DecodeArgs& p) {
  switch (p.Dv) {
    case 16: return launch_decode_t<TIn, TOut, DK, 16>(p);
    case 32: return launch_decode_t<TIn, TOut, DK, 32>(p);
    case 64: return launch_decode_t<TIn, TOut, DK, 64>(p);
    case 128: return launch_decode_t<TIn, TOut, DK, 128>(p);
  }
  return hipErrorInvalidValue;
}

template <class TIn, class TOut>
static hipError_t launch_decode_dk(const DecodeArgs& p) {
  switch (p.Dk) {
    case 16: return launch_decode_dv<TIn, TOut, 16>(p);
    case 32: return launch_decode_dv<TIn, TOut, 32>(p);
    case 64: return launch_decode_dv<TIn, TOut, 64>(p);
    case 128: return launch_decode_dv<TIn, TOut, 128>(p);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& p) {
  if (p.B * p.H == 0) return hipSuccess;
  if (!p.bf16) return launch_decode_dk<float, float>(p);
  return p.out_bf16 ? launch_decode_dk<bf16, bf16>(p) : launch_decode_dk<bf16, float>(p);
}

}  // namespace gdn
