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
// The columns of S and G evolve independently, so one work-group of 512
// threads takes one (b, h) and a slice of 32 state columns and holds that
// DK x 32 part of S and G (f32) in LDS.  A forward sweep stores the state
// entering every chunk of BCK = 32 tokens (the checkpoints); the backward
// sweep takes the chunks in reverse, recomputes the chunk's states from its
// checkpoint into a per-work-group buffer, and runs the adjoint over the
// chunk's tokens in reverse, reading S_{t-1} back from that buffer.  The
// buffer and the checkpoints are written and read by the same thread.
// Gradients that sum over all columns (dq, dk, dalpha, dbeta) are written as
// per-slice partials and summed in slice order by a second kernel.  All
// arithmetic is f32; this is the direct form of the adjoint (no chunked
// rewrite), sequential over tokens.
#include <algorithm>

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

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N a power of two up to 64); every lane
// of the group ends with the total.  Within a row of 16 lanes by DPP moves
// (quad swaps, then half-row and row mirrors), across rows by swizzles.
template <int N>
__device__ __forceinline__ float lane_sum(float x) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "power-of-two lane group");
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp_mov<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Work-group per (b, h, slice of DVS state columns): the columns of S and of
// its adjoint G evolve independently, so each work-group carries DK x DVS of
// both.  Per-token quantities that sum over all columns (dq, dk, dalpha,
// dbeta) are written per slice to `part` and summed by bwd_reduce_kernel
// (written directly when there is one slice).  Every matrix-vector product
// uses the whole work-group: NPC threads per column (reduction index
// interleaved, lanes of one group summed by shuffles) or NPR threads per row.
template <class TIn, int DK, int DV, int DVS>
__global__ __launch_bounds__(BNT) void gdn_bwd_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ state_in, const float* __restrict__ dout,
    const float* __restrict__ dstate_out, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dalpha, float* __restrict__ dbeta,
    float* __restrict__ dstate_in, int T, int H, float scale, float* __restrict__ ws,
    float* __restrict__ part) {
  constexpr int NS = DV / DVS;
  constexpr int LD = DVS + 1;
  constexpr int SZ = DK * DVS;
  constexpr int NPT = (SZ + BNT - 1) / BNT;               // state elements per thread
  constexpr int NPC = (BNT / DVS < DK) ? BNT / DVS : DK;  // threads per column
  constexpr int NPR = (BNT / DK < DVS) ? BNT / DK : DVS;  // threads per row
  __shared__ float S[DK * LD], G[DK * LD];
  // The current chunk's token inputs (k, q rows; the slice's v, dout columns).
  __shared__ float ck[BCK * DK], cq[BCK * DK], cv[BCK * DVS], cdo[BCK * DVS], ca[BCK], cb[BCK];
  __shared__ float pv[DVS], gv[DVS], Gv[DK], Pg[DK], red[2][BNT / 64][3];
  const int bh = blockIdx.x / NS, sl = blockIdx.x % NS, b = bh / H, h = bh % H;
  const int col0 = sl * DVS;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int NC = (T + BCK - 1) / BCK;
  float* ckpt = ws + (size_t)blockIdx.x * (NC + BCK) * SZ;  // NC checkpoints, BCK chunk states
  float* cbuf = ckpt + (size_t)NC * SZ;
  const size_t BTH = (size_t)gridDim.x / NS * T;  // token-heads
  float* pdq = part + ((size_t)sl * BTH) * DK;
  float* pdk = part + ((size_t)NS * BTH) * DK + ((size_t)sl * BTH) * DK;
  float* pda = part + ((size_t)2 * NS * BTH) * DK + (size_t)sl * BTH;
  float* pdb = pda + (size_t)NS * BTH;

  // y_j = sum_i M[i][j] x_i for the slice's columns (x in LDS, length DK).
  auto colsum = [&](const float* M, const float* x, float* y) {
    const int j = tid / NPC, pp = tid % NPC;
    if (j < DVS) {
      float acc = 0.f;
#pragma unroll
      for (int i = pp; i < DK; i += NPC) acc += M[i * LD + j] * x[i];
      acc = lane_sum<NPC>(acc);
      if (pp == 0) y[j] = acc;
    }
  };
  // y_i = sum_j M[i][j] x_j over the slice's columns; returns the sum in the
  // lane with pp == 0 of row i (other lanes: partial), row index via *row.
  auto rowsum = [&](const float* M, const float* x, int* row) {
    const int i = tid / NPR, pp = tid % NPR;
    *row = (i < DK && pp == 0) ? i : -1;
    float acc = 0.f;
    if (i < DK) {
#pragma unroll
      for (int j = pp; j < DVS; j += NPR) acc += M[i * LD + j] * x[j];
    }
    return lane_sum<NPR>(acc);
  };
  // Tokens [t0, t1) of the chunk into LDS (q and dout only when wanted).
  auto load_chunk = [&](int t0, int t1, bool with_q) {
    const int n = t1 - t0;
    const size_t row0 = ((size_t)b * T + t0) * H + h;
    for (int e = tid; e < n * DK; e += BNT) {
      const size_t off = (row0 + (size_t)(e / DK) * H) * DK + e % DK;
      ck[e] = ldin(k + off);
      if (with_q) cq[e] = ldin(q + off);
    }
    for (int e = tid; e < n * DVS; e += BNT) {
      const size_t off = (row0 + (size_t)(e / DVS) * H) * DV + col0 + e % DVS;
      cv[e] = ldin(v + off);
      if (with_q) cdo[e] = dout[off];
    }
    if (tid < n) {
      ca[tid] = alpha[row0 + (size_t)tid * H];
      cb[tid] = beta[row0 + (size_t)tid * H];
    }
  };
  auto step = [&](int tl) {  // S <- A_t S + beta_t k v^T, token tl of the chunk
    const float* kv = ck + tl * DK;
    const float* vv = cv + tl * DVS;
    __syncthreads();  // chunk inputs loaded, previous update done
    const float a = ca[tl], be = cb[tl];
    colsum(S, kv, pv);
    __syncthreads();
    for (int e = tid; e < SZ; e += BNT) {
      const int i = e / DVS, j = e % DVS;
      S[i * LD + j] = a * (S[i * LD + j] - be * kv[i] * pv[j]) + be * kv[i] * vv[j];
    }
  };
  auto save = [&](float* dst) {
    for (int e = tid; e < SZ; e += BNT) dst[e] = S[(e / DVS) * LD + e % DVS];
  };
  auto restore = [&](const float* src) {
    for (int e = tid; e < SZ; e += BNT) S[(e / DVS) * LD + e % DVS] = src[e];
  };
  // Per-wave partial sums of three values into red[par]; read after the
  // next barrier (red is double-buffered by token parity).
  auto wave_sum3 = [&](float x0, float x1, float x2, int par) {
    x0 = lane_sum<64>(x0);
    x1 = lane_sum<64>(x1);
    x2 = lane_sum<64>(x2);
    if (lane == 0) {
      red[par][wv][0] = x0;
      red[par][wv][1] = x1;
      red[par][wv][2] = x2;
    }
  };

  // Forward sweep: checkpoints.
  for (int e = tid; e < SZ; e += BNT)
    S[(e / DVS) * LD + e % DVS] =
        state_in ? state_in[((size_t)bh * DK + e / DVS) * DV + col0 + e % DVS] : 0.f;
  for (int c = 0; c < NC; ++c) {
    const int t0 = c * BCK, t1 = min(T, t0 + BCK);
    __syncthreads();  // previous chunk's last update done
    save(ckpt + (size_t)c * SZ);
    load_chunk(t0, t1, false);
    for (int t = t0; t < t1; ++t) step(t - t0);
  }

  // Backward sweep.
  for (int e = tid; e < SZ; e += BNT)
    G[(e / DVS) * LD + e % DVS] =
        dstate_out ? dstate_out[((size_t)bh * DK + e / DVS) * DV + col0 + e % DVS] : 0.f;
  for (int c = NC - 1; c >= 0; --c) {
    const int t0 = c * BCK, t1 = min(T, t0 + BCK);
    __syncthreads();  // previous chunk's last carry done, chunk buffers free
    restore(ckpt + (size_t)c * SZ);
    load_chunk(t0, t1, true);
    for (int t = t0; t < t1; ++t) {
      __syncthreads();
      save(cbuf + (size_t)(t - t0) * SZ);  // S_{t-1}
      step(t - t0);
    }
    for (int t = t1 - 1; t >= t0; --t) {
      const int tl = t - t0;
      const size_t row = ((size_t)b * T + t) * H + h;
      const float a = ca[tl], be = cb[tl];
      const float* kv = ck + tl * DK;
      const float* qv = cq + tl * DK;
      const float* vv = cv + tl * DVS;
      const float* dov = cdo + tl * DVS;
      // S_{t-1}, written by this thread in the recompute loop, fetched early.
      float prev[NPT];
#pragma unroll
      for (int u = 0; u < NPT; ++u) {
        const int e = tid + u * BNT;
        prev[u] = (e < SZ) ? cbuf[(size_t)tl * SZ + e] : 0.f;
      }
      __syncthreads();  // previous carry done
      for (int e = tid; e < SZ; e += BNT) {
        const int i = e / DVS, j = e % DVS;
        G[i * LD + j] += scale * qv[i] * dov[j];
      }
      __syncthreads();
      int ri;
      const float dqp = rowsum(S, dov, &ri);  // S_t do (this slice's columns)
      if (ri >= 0) (NS == 1 ? dq + row * DK : pdq + row * DK)[ri] = scale * dqp;
      const float gvp = rowsum(G, vv, &ri);
      if (ri >= 0) Gv[ri] = gvp;
      colsum(G, kv, gv);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NPT; ++u) {  // S <- S_{t-1}
        const int e = tid + u * BNT;
        if (e < SZ) S[(e / DVS) * LD + e % DVS] = prev[u];
      }
      __syncthreads();
      colsum(S, kv, pv);
      const float pg = rowsum(S, gv, &ri);
      if (ri >= 0) Pg[ri] = pg;
      float gP = 0.f;
      for (int e = tid; e < SZ; e += BNT) {
        const int i = e / DVS, j = e % DVS;
        gP += G[i * LD + j] * S[i * LD + j];
      }
      __syncthreads();  // pv, Pg ready
      float gpp = 0.f, gvv = 0.f;
      if (tid < DVS) {
        gpp = gv[tid] * pv[tid];
        gvv = gv[tid] * (vv[tid] - a * pv[tid]);
        dv[row * DV + col0 + tid] = be * gv[tid];
      }
      const float gp = rowsum(G, pv, &ri);
      if (ri >= 0)
        (NS == 1 ? dk + row * DK : pdk + row * DK)[ri] = -a * be * (gp + Pg[ri]) + be * Gv[ri];
      wave_sum3(gP, gpp, gvv, t & 1);
      __syncthreads();  // G reads and wave partials done
      if (tid == 0) {
        float s0 = 0.f, s1 = 0.f, s2 = 0.f;
        for (int w = 0; w < BNT / 64; ++w) {
          s0 += red[t & 1][w][0];
          s1 += red[t & 1][w][1];
          s2 += red[t & 1][w][2];
        }
        (NS == 1 ? dalpha + row : pda + row)[0] = s0 - be * s1;
        (NS == 1 ? dbeta + row : pdb + row)[0] = s2;
      }
      // Carry: G <- A_t G.
      for (int e = tid; e < SZ; e += BNT) {
        const int i = e / DVS, j = e % DVS;
        G[i * LD + j] = a * (G[i * LD + j] - be * kv[i] * gv[j]);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < SZ; e += BNT)
    dstate_in[((size_t)bh * DK + e / DVS) * DV + col0 + e % DVS] = G[(e / DVS) * LD + e % DVS];
}

// Sums the per-slice partials of dq, dk, dalpha, dbeta (NS slices).
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ part,
                                                         float* __restrict__ dq,
                                                         float* __restrict__ dk,
                                                         float* __restrict__ dalpha,
                                                         float* __restrict__ dbeta, size_t BTH,
                                                         int DK, int NS) {
  const size_t n = BTH * DK;
  const float* pdq = part;
  const float* pdk = part + (size_t)NS * n;
  const float* pda = part + (size_t)2 * NS * n;
  const float* pdb = pda + (size_t)NS * BTH;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) {
    float a = 0.f, c = 0.f;
    for (int s2 = 0; s2 < NS; ++s2) {
      a += pdq[(size_t)s2 * n + e];
      c += pdk[(size_t)s2 * n + e];
    }
    dq[e] = a;
    dk[e] = c;
  }
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < BTH; e += (size_t)gridDim.x * 256) {
    float a = 0.f, c = 0.f;
    for (int s2 = 0; s2 < NS; ++s2) {
      a += pda[(size_t)s2 * BTH + e];
      c += pdb[(size_t)s2 * BTH + e];
    }
    dalpha[e] = a;
    dbeta[e] = c;
  }
}

constexpr int kBwdSlice = 32;  // state columns per work-group

template <class TIn, int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs& p) {
  constexpr int DVS = DV < kBwdSlice ? DV : kBwdSlice;
  constexpr int NS = DV / DVS;
  const int NC = (p.T + BCK - 1) / BCK;
  float* ws = (float*)p.workspace;
  float* part = ws + (size_t)p.B * p.H * NS * (NC + BCK) * DK * DVS;
  const hipStream_t st = (hipStream_t)p.stream;
  hipLaunchKernelGGL((gdn_bwd_kernel<TIn, DK, DV, DVS>), dim3(p.B * p.H * NS), dim3(BNT), 0, st,
                     (const TIn*)p.q, (const TIn*)p.k, (const TIn*)p.v, p.alpha, p.beta,
                     p.state_in, p.dout, p.dstate_out, p.dq, p.dk, p.dv, p.dalpha, p.dbeta,
                     p.dstate_in, p.T, p.H, p.scale, ws, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || NS == 1 || p.T == 0) return e;
  const size_t BTH = (size_t)p.B * p.T * p.H;
  const unsigned blocks = (unsigned)std::min<size_t>((BTH * DK + 255) / 256, 4096);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(blocks), dim3(256), 0, st, part, p.dq, p.dk,
                     p.dalpha, p.dbeta, BTH, DK, NS);
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
  const size_t dvs = Dv < kBwdSlice ? Dv : kBwdSlice, ns = Dv / dvs;
  const size_t ckpt = (size_t)B * H * ns * (nc + BCK) * Dk * dvs;
  const size_t part = ns > 1 ? ns * (size_t)B * T * H * (2 * (size_t)Dk + 2) : 0;
  return (ckpt + part) * sizeof(float);
}

hipError_t launch_backward(const BwdArgs& p) {
  if ((long long)p.B * p.H == 0) return hipSuccess;
  return p.bf16 ? launch_bwd_dk<bf16>(p) : launch_bwd_dk<float>(p);
}

}  // namespace gdn
