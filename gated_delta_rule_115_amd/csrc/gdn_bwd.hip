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
// The columns of S and G evolve independently, so one work-group takes one
// (b, h) and a slice of 32 state columns (16 when Dv = 16) and holds that
// Dk x 32 part of S and G (f32) in registers, 16 lanes per column.  A forward
// sweep stores the state entering every SUB = 4th token (the checkpoints);
// the backward sweep takes the tokens in reverse, SUB at a time: it
// recomputes the states entering those tokens from their checkpoint into
// registers and runs the adjoint over them.  Token inputs are staged in LDS
// BCK = 32 tokens at a time.  Gradients that sum over all columns (dq, dk,
// dalpha, dbeta) are written as per-slice partials and summed in slice order
// by a second kernel.  All arithmetic is f32; this is the direct form of the
// adjoint (no chunked rewrite), sequential over tokens.
#include <algorithm>

#include "gdn_device.h"
#include "gdn_f16ops.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int BCK = 32;  // tokens staged in LDS at a time
constexpr int SUB = 4;  // tokens per checkpoint (states recomputed into registers)
static_assert(BCK % SUB == 0, "checkpoints fall on sub-chunk starts within a staged chunk");

template <class TIn>
__device__ __forceinline__ float ldin(const TIn* p) {
  return to_f32(*p);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Value of lane (lane ^ 16): ds_swizzle in bit-mask mode within 32-lane
// halves (and mask 0x1F, or mask 0, xor mask 0x10).
__device__ __forceinline__ float xor16(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}
// Value of lane (lane ^ 32); a32 = ((lane ^ 32) << 2), computed once.
__device__ __forceinline__ float xor32(float x, int a32) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_bpermute(a32, __builtin_bit_cast(int, x)));
}

// Sum over aligned groups of N lanes (N a power of two up to 64); every lane
// of the group ends with the total.  Within a row of 16 lanes by DPP moves
// (quad swaps, then half-row and row mirrors), across rows by a swizzle and
// a permute.
template <int N>
__device__ __forceinline__ float lane_sum(float x, int a32 = 0) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "power-of-two lane group");
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp_mov<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += xor16(x);
  if constexpr (N >= 64) x += xor32(x, a32);
  return x;
}

// Work-group per (b, h, slice of DVS state columns): the columns of S and of
// its adjoint G evolve independently, so each work-group carries DK x DVS of
// both.  Per-token quantities that sum over all columns (dq, dk, dalpha,
// dbeta) are written per slice to `part` and summed by bwd_reduce_kernel
// (written directly when there is one slice).  Every matrix-vector product
// uses the whole work-group: NPC threads per column (reduction index
// interleaved, lanes of one group summed by shuffles) or NPR threads per row.
// Sum over the four 16-lane column groups of a wave of R per-lane row
// values x[u] (rows pp*R + u), written as the wave's partial to dst[row].
// For R >= 4 it is a reduce-scatter (halving over lane bit 5, then bit 4);
// each row is written by exactly one lane.
template <int R>
__device__ __forceinline__ void wave_rows_to_lds(const float (&x)[R], int lane, int pp, int a32,
                                                 float* dst) {
  const bool b5 = lane & 32, b4 = lane & 16;
  if constexpr (R >= 4) {
    float y[R / 2], z[R / 4];
#pragma unroll
    for (int m = 0; m < R / 2; ++m) {
      const float send = b5 ? x[m] : x[m + R / 2];
      y[m] = (b5 ? x[m + R / 2] : x[m]) + xor32(send, a32);
    }
#pragma unroll
    for (int m = 0; m < R / 4; ++m) {
      const float send = b4 ? y[m] : y[m + R / 4];
      z[m] = (b4 ? y[m + R / 4] : y[m]) + xor16(send);
    }
    const int u0 = (b5 ? R / 2 : 0) + (b4 ? R / 4 : 0);
#pragma unroll
    for (int m = 0; m < R / 4; ++m) dst[pp * R + u0 + m] = z[m];
  } else if constexpr (R == 2) {
    float y = (b5 ? x[1] : x[0]) + xor32(b5 ? x[0] : x[1], a32);
    y += xor16(y);
    if (!b4) dst[pp * 2 + (b5 ? 1 : 0)] = y;
  } else {
    float y = x[0] + xor32(x[0], a32);
    y += xor16(y);
    if (lane < 16) dst[pp] = y;
  }
}

// Thread layout: 16 lanes per state column (a DPP row), DVS columns, so
// NT = 16 * DVS threads; lane pp of column j holds rows pp*RPT .. pp*RPT+RPT-1
// of that column of S and of G in registers.  Column sums (S^T k, G^T k) are
// 16-lane DPP sums; row sums (dq, dk) go through a per-wave reduce-scatter and
// an LDS array double-buffered by token parity, so the backward token loop
// has one barrier per token and the forward steps none.
template <class TIn, int DK, int DV, int DVS>
__global__ __launch_bounds__(512) void gdn_bwd_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ state_in, const float* __restrict__ dout,
    const float* __restrict__ dstate_out, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dalpha, float* __restrict__ dbeta,
    float* __restrict__ dstate_in, int T, int H, float scale, float* __restrict__ ws,
    float* __restrict__ part) {
  constexpr int NS = DV / DVS;
  constexpr int NT = 16 * DVS;
  constexpr int NW = NT / 64;
  constexpr int RPT = DK / 16;
  constexpr int SZ = DK * DVS;
  static_assert(NT * RPT == SZ && NT <= 512, "thread layout");
  // The current chunk's token inputs (k, q rows; the slice's v, dout columns).
  __shared__ float ck[BCK * DK], cq[BCK * DK], cv[BCK * DVS], cdo[BCK * DVS], ca[BCK], cb[BCK];
  __shared__ float rowp[2][2][NW][DK], scal[2][NW][2];
  const int bh = blockIdx.x / NS, sl = blockIdx.x % NS, b = bh / H, h = bh % H;
  const int col0 = sl * DVS;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int j = tid >> 4, pp = tid & 15, r0 = pp * RPT;
  const int a32 = (lane ^ 32) << 2;  // byte address of lane ^ 32 for ds_bpermute
  const int NC = (T + BCK - 1) / BCK;
  float* ckpt = ws + (size_t)blockIdx.x * ((T + SUB - 1) / SUB) * SZ;  // one per SUB tokens
  const size_t BTH = (size_t)gridDim.x / NS * T;  // token-heads
  float* pdq = part + ((size_t)sl * BTH) * DK;
  float* pdk = part + ((size_t)NS * BTH) * DK + ((size_t)sl * BTH) * DK;
  float* pda = part + ((size_t)2 * NS * BTH) * DK + (size_t)sl * BTH;
  float* pdb = pda + (size_t)NS * BTH;
  const size_t sbase = (size_t)bh * DK * DV + col0 + j;  // element (r0, j) of a [DK, DV] state

  float S[RPT], G[RPT];
  // Tokens [t0, t1) of the chunk into LDS (q and dout only when wanted).
  // Every thread issues a fixed number of loads, all before the first LDS
  // store; slots past the chunk's last token repeat that token.
  constexpr int KE = BCK * DK / NT, VE = BCK * DVS / NT;
  static_assert(KE * NT == BCK * DK && VE * NT == BCK * DVS && BCK <= NT, "chunk staging");
  auto load_chunk = [&](int t0, int t1, bool with_q) {
    const int last = t1 - t0 - 1;
    const size_t row0 = ((size_t)b * T + t0) * H + h;
    float kr[KE], qr[KE], vr[VE], dr[VE];
#pragma unroll
    for (int u = 0; u < KE; ++u) {
      const int e = tid + u * NT;
      const size_t off = (row0 + (size_t)min(e / DK, last) * H) * DK + e % DK;
      kr[u] = ldin(k + off);
      if (with_q) qr[u] = ldin(q + off);
    }
#pragma unroll
    for (int u = 0; u < VE; ++u) {
      const int e = tid + u * NT;
      const size_t off = (row0 + (size_t)min(e / DVS, last) * H) * DV + col0 + e % DVS;
      vr[u] = ldin(v + off);
      if (with_q) dr[u] = dout[off];
    }
    float ar = 0.f, br = 0.f;
    if (tid < BCK) {
      ar = alpha[row0 + (size_t)min(tid, last) * H];
      br = beta[row0 + (size_t)min(tid, last) * H];
    }
#pragma unroll
    for (int u = 0; u < KE; ++u) {
      ck[tid + u * NT] = kr[u];
      if (with_q) cq[tid + u * NT] = qr[u];
    }
#pragma unroll
    for (int u = 0; u < VE; ++u) {
      cv[tid + u * NT] = vr[u];
      if (with_q) cdo[tid + u * NT] = dr[u];
    }
    if (tid < BCK) {
      ca[tid] = ar;
      cb[tid] = br;
    }
  };
  // dst <- A_t src + beta_t k v^T for token tl of the chunk (dst may be src).
  auto step = [&](int tl, const float (&src)[RPT], float (&dst)[RPT]) {
    const float a = ca[tl], be = cb[tl], vj = cv[tl * DVS + j];
    float kk[RPT], acc = 0.f;
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      kk[u] = ck[tl * DK + r0 + u];
      acc += src[u] * kk[u];
    }
    // a (S - be k p^T) + be k v^T = a S + k (be (v - a p))^T
    const float cj = be * (vj - a * lane_sum<16>(acc));
#pragma unroll
    for (int u = 0; u < RPT; ++u) dst[u] = fmaf(kk[u], cj, a * src[u]);
  };
  auto save = [&](float* dst) {
#pragma unroll
    for (int u = 0; u < RPT; ++u) dst[u * NT + tid] = S[u];
  };

  // One token of the adjoint, token tl of the staged chunk, with St = S_t and
  // P = S_{t-1}; leaves G = A_t G_t.
  auto adjoint = [&](int t, int tl, const float (&St)[RPT], const float (&P)[RPT]) {
    const int par = t & 1;
    const size_t row = ((size_t)b * T + t) * H + h;
    const float a = ca[tl], be = cb[tl];
    const float vj = cv[tl * DVS + j], doj = cdo[tl * DVS + j];
    float kk[RPT], rq[RPT], rk[RPT];
    float gacc = 0.f;
    const float sdo = scale * doj;
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      kk[u] = ck[tl * DK + r0 + u];
      G[u] = fmaf(cq[tl * DK + r0 + u], sdo, G[u]);  // G_t
      rq[u] = St[u] * doj;                           // S_t do (row sums give dq / scale)
      gacc = fmaf(G[u], kk[u], gacc);
    }
    const float gj = lane_sum<16>(gacc);  // (G_t^T k)_j
    float pacc = 0.f;
#pragma unroll
    for (int u = 0; u < RPT; ++u) pacc = fmaf(P[u], kk[u], pacc);
    const float pj = lane_sum<16>(pacc);  // (S_{t-1}^T k)_j
    // dk row terms: -a be (G p + P g) + be G v = G (be (v - a p)) + P (-a be g)
    const float c1 = be * (vj - a * pj), c2 = -a * be * gj;
    float sA = 0.f;
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      rk[u] = fmaf(G[u], c1, P[u] * c2);
      sA = fmaf(G[u], P[u], sA);
    }
    float sB = 0.f;
    if (pp == 0) {
      sA -= be * gj * pj;
      sB = gj * (vj - a * pj);
      dv[row * DV + col0 + j] = be * gj;
    }
    wave_rows_to_lds<RPT>(rq, lane, pp, a32, rowp[par][0][wv]);
    wave_rows_to_lds<RPT>(rk, lane, pp, a32, rowp[par][1][wv]);
    sA = lane_sum<64>(sA, a32);
    sB = lane_sum<64>(sB, a32);
    if (lane == 0) {
      scal[par][wv][0] = sA;
      scal[par][wv][1] = sB;
    }
#pragma unroll
    for (int u = 0; u < RPT; ++u) G[u] = fmaf(kk[u], c2, a * G[u]);  // A_t G_t
    f16ops::lds_barrier();  // wave partials of token t complete
    if (tid < DK) {
      float x = 0.f, y = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        x += rowp[par][0][w][tid];
        y += rowp[par][1][w][tid];
      }
      (NS == 1 ? dq : pdq)[row * DK + tid] = scale * x;
      (NS == 1 ? dk : pdk)[row * DK + tid] = y;
    } else if (tid == DK) {
      float x = 0.f, y = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        x += scal[par][w][0];
        y += scal[par][w][1];
      }
      (NS == 1 ? dalpha : pda)[row] = x;
      (NS == 1 ? dbeta : pdb)[row] = y;
    }
  };

  // Forward sweep: the state entering every SUB-th token is checkpointed.
#pragma unroll
  for (int u = 0; u < RPT; ++u) S[u] = state_in ? state_in[sbase + (size_t)(r0 + u) * DV] : 0.f;
  for (int c = 0; c < NC; ++c) {
    const int t0 = c * BCK, t1 = min(T, t0 + BCK);
    f16ops::lds_barrier();  // previous chunk's reads of the chunk buffers done
    load_chunk(t0, t1, false);
    f16ops::lds_barrier();
    for (int t = t0; t < t1; ++t) {
      if (t % SUB == 0) save(ckpt + (size_t)(t / SUB) * SZ);
      step(t - t0, S, S);
    }
  }

  // Backward sweep: chunks of BCK tokens staged in LDS, in reverse; within
  // a chunk, sub-chunks of SUB tokens in reverse: the states entering the
  // sub-chunk's tokens are recomputed from its checkpoint into registers
  // (hist), then the adjoint runs over them.  The checkpoint of the next
  // sub-chunk is fetched while the current one is processed.
#pragma unroll
  for (int u = 0; u < RPT; ++u)
    G[u] = dstate_out ? dstate_out[sbase + (size_t)(r0 + u) * DV] : 0.f;
  const int NCK = (T + SUB - 1) / SUB;  // 0 when T = 0: no checkpoint to read
  float nxt[RPT] = {};
  if (NCK > 0) {
#pragma unroll
    for (int u = 0; u < RPT; ++u) nxt[u] = ckpt[(size_t)(NCK - 1) * SZ + u * NT + tid];
  }
  for (int c = NC - 1; c >= 0; --c) {
    const int t0 = c * BCK, t1 = min(T, t0 + BCK);
    f16ops::lds_barrier();  // previous chunk's reads of the chunk buffers done
    load_chunk(t0, t1, true);
    f16ops::lds_barrier();
    for (int s0 = t0 + ((t1 - 1 - t0) / SUB) * SUB; s0 >= t0; s0 -= SUB) {
      const int n = min(SUB, t1 - s0), ci = s0 / SUB;
      float hist[SUB + 1][RPT];  // hist[i]: the state entering token s0 + i
#pragma unroll
      for (int u = 0; u < RPT; ++u) {
        hist[0][u] = nxt[u];
        nxt[u] = ckpt[(size_t)max(ci - 1, 0) * SZ + u * NT + tid];
      }
#pragma unroll
      for (int i = 0; i < SUB; ++i)
        if (i < n) step(s0 + i - t0, hist[i], hist[i + 1]);
#pragma unroll
      for (int i = SUB - 1; i >= 0; --i)
        if (i < n) adjoint(s0 + i, s0 + i - t0, hist[i + 1], hist[i]);
    }
  }
#pragma unroll
  for (int u = 0; u < RPT; ++u) dstate_in[sbase + (size_t)(r0 + u) * DV] = G[u];
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
  const int NCK = (p.T + SUB - 1) / SUB;
  float* ws = (float*)p.workspace;
  float* part = ws + (size_t)p.B * p.H * NS * NCK * DK * DVS;
  const hipStream_t st = (hipStream_t)p.stream;
  hipLaunchKernelGGL((gdn_bwd_kernel<TIn, DK, DV, DVS>), dim3(p.B * p.H * NS), dim3(16 * DVS), 0, st,
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
  if (backward_chunked_supported(Dk, Dv)) return backward_chunked_workspace_bytes(B, T, H);
  const size_t nck = ((size_t)T + SUB - 1) / SUB;
  const size_t dvs = Dv < kBwdSlice ? Dv : kBwdSlice, ns = Dv / dvs;
  const size_t ckpt = (size_t)B * H * ns * nck * Dk * dvs;
  const size_t part = ns > 1 ? ns * (size_t)B * T * H * (2 * (size_t)Dk + 2) : 0;
  return (ckpt + part) * sizeof(float);
}

hipError_t launch_backward(const BwdArgs& p) {
  if ((long long)p.B * p.H == 0) return hipSuccess;
  if (backward_chunked_supported(p.Dk, p.Dv)) return launch_backward_chunked(p);
  return p.bf16 ? launch_bwd_dk<bf16>(p) : launch_bwd_dk<float>(p);
}

}  // namespace gdn
