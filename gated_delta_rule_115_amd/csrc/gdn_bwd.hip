// Backward pass of the GDN recurrence (scalar gate), gfx950.
//
// "The Key to Going Linear: Analysis-Driven Transformer Linearization",
// section 3.1.2: S_t = A_t S_{t-1} + beta_t k_t v_t^T with
// A_t = alpha_t (I - beta_t k_t k_t^T) (symmetric) and o_t = scale S_t^T q_t;
// section 3.3 trains the gate and step-size projections through the mixer.
// The adjoint of the token loop: the total gradient G_t = dL/dS_t obeys
//   G_t = scale q_t do_t^T + A_{t+1} G_{t+1}   (G at the last token starts
//   from the final-state gradient),
// and with P = S_{t-1}, p = P^T k_t, g = G_t^T k_t:
//   dq_t = scale S_t do_t,  dv_t = beta_t g,
//   dalpha_t = <G_t, P> - beta_t g.p,  dbeta_t = g.(v_t - alpha_t p),
//   dk_t = -alpha_t beta_t (G_t p + P g) + beta_t G_t v_t,
//   and the initial-state gradient is A_0 G_0.
//
// One work-group of 512 threads per (b, h) holds S and G (f32) in LDS.  A
// forward sweep stores the state entering every chunk of BCK = 32 tokens
// (the checkpoints); the backward sweep takes the chunks in reverse, recomputes
// the chunk's states from its checkpoint into a per-head buffer, and runs
// the adjoint over the chunk's tokens in reverse, reading S_{t-1} back from
// that buffer.  The buffer is written and read by the same work-group across
// full barriers.  All arithmetic is f32; this is the direct form of the
// adjoint (no chunked rewrite), sequential over tokens.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int BCK = 32;   // tokens per checkpointed chunk
constexpr int BNT = 512;  // threads per work-group

template <class TIn>
__device__ __forceinline__ float ldin(const TIn* p) {
  return to_f32(*p);
}

template <class TIn, int DK, int DV>
__global__ __launch_bounds__(BNT) void gdn_bwd_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ state_in, const float* __restrict__ dout,
    const float* __restrict__ dstate_out, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dalpha, float* __restrict__ dbeta,
    float* __restrict__ dstate_in, int T, int H, float scale, float* __restrict__ ws) {
  constexpr int LD = DV + 1;
  constexpr int SZ = DK * DV;
  __shared__ float S[DK * LD], G[DK * LD];
  __shared__ float kv[DK], qv[DK], vv[DV], dov[DV];
  __shared__ float pv[DV], gv[DV], Gv[DK], Pg[DK], red[BNT / 64][3], sc[3];
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int NC = (T + BCK - 1) / BCK;
  float* ckpt = ws + (size_t)bh * (NC + BCK) * SZ;  // NC checkpoints, then BCK chunk states
  float* cbuf = ckpt + (size_t)NC * SZ;

  auto load_tok = [&](int t) {  // k, q, v, do of token t into LDS
    const size_t row = ((size_t)b * T + t) * H + h;
    for (int i = tid; i < DK; i += BNT) {
      kv[i] = ldin(k + row * DK + i);
      qv[i] = ldin(q + row * DK + i);
    }
    for (int j = tid; j < DV; j += BNT) {
      vv[j] = ldin(v + row * DV + j);
      dov[j] = dout[row * DV + j];
    }
  };
  auto step = [&](int t) {  // S <- A_t S + beta_t k v^T
    const size_t row = ((size_t)b * T + t) * H + h;
    const float a = alpha[row], be = beta[row];
    __syncthreads();  // kv, vv of token t visible
    if (tid < DV) {
      float acc = 0.f;
      for (int i = 0; i < DK; ++i) acc += S[i * LD + tid] * kv[i];
      pv[tid] = acc;
    }
    __syncthreads();
    for (int e = tid; e < SZ; e += BNT) {
      const int i = e / DV, j = e % DV;
      S[i * LD + j] = a * (S[i * LD + j] - be * kv[i] * pv[j]) + be * kv[i] * vv[j];
    }
  };
  auto save = [&](float* dst) {  // S -> dst (dense DK x DV)
    for (int e = tid; e < SZ; e += BNT) dst[e] = S[(e / DV) * LD + e % DV];
  };
  auto restore = [&](const float* src) {
    for (int e = tid; e < SZ; e += BNT) S[(e / DV) * LD + e % DV] = src[e];
  };
  // Sums over the work-group of three values per thread (into sc).
  auto block_sum3 = [&](float x0, float x1, float x2) {
    for (int off = 32; off > 0; off >>= 1) {
      x0 += __shfl_xor(x0, off);
      x1 += __shfl_xor(x1, off);
      x2 += __shfl_xor(x2, off);
    }
    if (lane == 0) {
      red[wv][0] = x0;
      red[wv][1] = x1;
      red[wv][2] = x2;
    }
    __syncthreads();
    if (tid < 3) {
      float s = 0.f;
      for (int w = 0; w < BNT / 64; ++w) s += red[w][tid];
      sc[tid] = s;
    }
    __syncthreads();
  };

  // Forward sweep: checkpoints.
  for (int e = tid; e < SZ; e += BNT)
    S[(e / DV) * LD + e % DV] = state_in ? state_in[(size_t)bh * SZ + e] : 0.f;
  __syncthreads();
  for (int c = 0; c < NC; ++c) {
    save(ckpt + (size_t)c * SZ);
    for (int t = c * BCK; t < min(T, (c + 1) * BCK); ++t) {
      __syncthreads();
      load_tok(t);
      step(t);
    }
    __syncthreads();
  }

  // Backward sweep.
  for (int e = tid; e < SZ; e += BNT)
    G[(e / DV) * LD + e % DV] = dstate_out ? dstate_out[(size_t)bh * SZ + e] : 0.f;
  for (int c = NC - 1; c >= 0; --c) {
    const int t0 = c * BCK, t1 = min(T, t0 + BCK);
    __syncthreads();
    restore(ckpt + (size_t)c * SZ);
    for (int t = t0; t < t1; ++t) {
      __syncthreads();
      save(cbuf + (size_t)(t - t0) * SZ);  // S_{t-1}
      load_tok(t);
      step(t);
    }
    // S holds S_{t1-1}.
    for (int t = t1 - 1; t >= t0; --t) {
      const size_t row = ((size_t)b * T + t) * H + h;
      const float a = alpha[row], be = beta[row];
      __syncthreads();
      load_tok(t);
      __syncthreads();
      // G_t = scale q do^T + (carried part)
      for (int e = tid; e < SZ; e += BNT) {
        const int i = e / DV, j = e % DV;
        G[i * LD + j] += scale * qv[i] * dov[j];
      }
      __syncthreads();
      // dq = scale S_t do (threads 0..DK-1), G v (threads 128..128+DK-1) and
      // g = G^T k (threads 256..256+DV-1) side by side.
      if (tid < DK) {
        float acc = 0.f;
        for (int j = 0; j < DV; ++j) acc += S[tid * LD + j] * dov[j];
        dq[row * DK + tid] = scale * acc;
      } else if (tid >= 128 && tid < 128 + DK) {
        const int i = tid - 128;
        float acc = 0.f;
        for (int j = 0; j < DV; ++j) acc += G[i * LD + j] * vv[j];
        Gv[i] = acc;
      } else if (tid >= 256 && tid < 256 + DV) {
        const int j = tid - 256;
        float acc = 0.f;
        for (int i = 0; i < DK; ++i) acc += G[i * LD + j] * kv[i];
        gv[j] = acc;
      }
      __syncthreads();
      // S <- S_{t-1} (P).
      restore(cbuf + (size_t)(t - t0) * SZ);
      __syncthreads();
      // p = P^T k (threads 0..DV-1), P g (threads 256..256+DK-1).
      if (tid < DV) {
        float acc = 0.f;
        for (int i = 0; i < DK; ++i) acc += S[i * LD + tid] * kv[i];
        pv[tid] = acc;
      } else if (tid >= 256 && tid < 256 + DK) {
        const int i = tid - 256;
        float acc = 0.f;
        for (int j = 0; j < DV; ++j) acc += S[i * LD + j] * gv[j];
        Pg[i] = acc;
      }
      float part = 0.f;  // <G, P>
      for (int e = tid; e < SZ; e += BNT) {
        const int i = e / DV, j = e % DV;
        part += G[i * LD + j] * S[i * LD + j];
      }
      __syncthreads();  // pv, Pg ready
      float gpp = 0.f, gvp = 0.f;
      if (tid < DV) {
        gpp = gv[tid] * pv[tid];
        gvp = gv[tid] * (vv[tid] - a * pv[tid]);
        dv[row * DV + tid] = be * gv[tid];
      }
      block_sum3(part, gpp, gvp);
      if (tid == 0) {
        dalpha[row] = sc[0] - be * sc[1];
        dbeta[row] = sc[2];
      }
      // dk = -a be (G p + P g) + be G v (threads 0..DK-1; G p here).
      if (tid < DK) {
        float acc = 0.f;
        for (int j = 0; j < DV; ++j) acc += G[tid * LD + j] * pv[j];
        dk[row * DK + tid] = -a * be * (acc + Pg[tid]) + be * Gv[tid];
      }
      __syncthreads();
      // Carry: G <- A_t G = a (G - be k g^T).
      for (int e = tid; e < SZ; e += BNT) {
        const int i = e / DV, j = e % DV;
        G[i * LD + j] = a * (G[i * LD + j] - be * kv[i] * gv[j]);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < SZ; e += BNT) dstate_in[(size_t)bh * SZ + e] = G[(e / DV) * LD + e % DV];
}

template <class TIn, int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs& p) {
  hipLaunchKernelGGL((gdn_bwd_kernel<TIn, DK, DV>), dim3(p.B * p.H), dim3(BNT), 0,
                     (hipStream_t)p.stream, (const TIn*)p.q, (const TIn*)p.k, (const TIn*)p.v,
                     p.alpha, p.beta, p.state_in, p.dout, p.dstate_out, p.dq, p.dk, p.dv,
                     p.dalpha, p.dbeta, p.dstate_in, p.T, p.H, p.scale, (float*)p.workspace);
  return hipGetLastError();
}

template <class TIn, int DK>
hipError_t launch_bwd_dv(const BwdArgs& p) {
  switch (p.Dv) {
    case 16: return launch_bwd_t<TIn, DK, 16>(p);
    case 32: return launch_bwd_t<TIn, DK, 32>(p);
    case 64: return launch_bwd_t<TIn, DK, 64>(p);
    case 128: return launch_bwd_t<TIn, DK, 128>(p);
  }
  return hipErrorInvalidValue;
}

template <class TIn>
hipError_t launch_bwd_dk(const BwdArgs& p) {
  switch (p.Dk) {
    case 16: return launch_bwd_dv<TIn, 16>(p);
    case 32: return launch_bwd_dv<TIn, 32>(p);
    case 64: return launch_bwd_dv<TIn, 64>(p);
    case 128: return launch_bwd_dv<TIn, 128>(p);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t backward_workspace_bytes(int B, int T, int H, int Dk, int Dv) {
  const size_t nc = ((size_t)T + BCK - 1) / BCK;
  return (size_t)B * H * (nc + BCK) * Dk * Dv * sizeof(float);
}

hipError_t launch_backward(const BwdArgs& p) {
  if ((long long)p.B * p.H == 0) return hipSuccess;
  return p.bf16 ? launch_bwd_dk<bf16>(p) : launch_bwd_dk<float>(p);
}

}  // namespace gdn
