// Chunked backward pass of the scalar-gate GDN prefill, gfx950, d_k = d_v = 128,
// chunks of C = 64 tokens, all arithmetic in f32 (v_mfma_f32_16x16x4_f32 for
// every product, f32 accumulation).
//
// "The Key to Going Linear: Analysis-Driven Transformer Linearization",
// section 3.1.2 (S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
// o_t = scale S_t^T q_t), trained through as in section 3.3.  The forward
// chunk form (gam_r = cumulative log gate from the chunk start, g_r =
// exp(gam_r), d_r = exp(gam_{C-1} - gam_r), G_ri = exp(gam_r - gam_i), S the
// state entering the chunk):
//   A_ri = beta_r G_ri k_r.k_i (i < r),  Tm = (I + A)^-1
//   Vm = V - diag(g) K S,  Y = diag(beta) Vm,  U = Tm Y
//   O = diag(scale g) Q S + P U,  P_ri = scale G_ri q_r.k_i (i <= r)
//   S_next = g_{C-1} S + K^T diag(d) U
// Its reverse mode, for the output gradient dO of the chunk and the gradient
// dSn of S_next:
//   dU = P^T dO + diag(d) K dSn,  dY = Tm^T dU,  dV = diag(beta) dY,
//   dX = -diag(beta g) dY,
//   dS = g_{C-1} dSn + Q^T diag(scale g) dO + K^T dX   (gradient of S),
//   dq = diag(scale g) dO S^T + E1 K,
//   dk = dX S^T + diag(d) U dSn^T + E1^T Q + (E2 + E2^T) K,
//   with dP = lower(dO U^T), E1 = scale G o dP, dA = -lower_strict(Tm^T dTm Tm^T),
//   dTm = dU Y^T, E2 = diag(beta) (G o dA);
//   dbeta_r = dY_r.Vm_r + sum_i dA_ri G_ri k_r.k_i;
//   dgam_r = dq_S,r.q_r + (dX S^T)_r.k_r - (diag(d) U dSn^T)_r.k_r
//            + sum_i (F_ri - F_ir),  F = dP o P + dA o A,
//   plus, on the last row, g_{C-1} <dSn, S> + sum_r (diag(d) U dSn^T)_r.k_r;
//   dlog(alpha_j) = sum_{r >= j} dgam_r and dalpha_j = dlog(alpha_j) / alpha_j.
// Only the dS chain is sequential over chunks; it needs neither S nor U.
//
// Four launches:
//   prep     (work-group per (b, h, chunk)): gam, Tm (diagonal 16 x 16 blocks
//            by forward substitution, the rest by block substitution), P and
//            the key Gram matrix K K^T, to a per-chunk record;
//   forward  (work-group per (b, h, value slice of 64 columns, 32 with f32
//            inputs), sequential): S entering every chunk, Vm and U of every
//            chunk;
//   dstate   (work-group per (b, h, value slice), sequential in reverse):
//            dSn of every chunk, dU and dY; dv, and dstate_in at the end;
//   grads    (work-group per (b, h, chunk)): everything else, over the full
//            value dimension (four 32-column passes), so dq, dk, dalpha and
//            dbeta are written once, with no partial sums.
// Ragged tails: rows past T read as alpha = 1, beta = 0, q = k = v = dO = 0,
// exact no-ops of the forward map, whose gradients vanish; the grads pass
// still runs its reverse sum of dgam over them (the last row's terms sit on
// row C - 1) and stores only rows before T.
#include <algorithm>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int C = 64;    // chunk
constexpr int D = 128;   // d_k = d_v
constexpr int QV = 32;   // value columns per pass of the grads kernel
constexpr int LC = C + 4;  // f32 row stride of C-wide tiles read k-contiguous

// Per-chunk record of the prep kernel (f32): Tm [C][C], P [C][C] (zero above
// the diagonal), Gk = K K^T [C][C] (zero on and above it), gam [C].
constexpr int REC = 3 * C * C + C;
// Workspace floats per (b, h, chunk): record, S and dSn [D][D] ([key][column]),
// Vm, U, dU, dY [C][D] ([token][column]).
constexpr size_t PER_CHUNK = (size_t)REC + 2 * D * D + 4 * C * D;

struct Ws {
  float *rec, *S, *dS, *Vm, *U, *dU, *dY;
};
__host__ __device__ inline Ws ws_split(float* base, size_t n) {
  Ws w;
  w.rec = base;
  w.S = w.rec + n * REC;
  w.dS = w.S + n * D * D;
  w.Vm = w.dS + n * D * D;
  w.U = w.Vm + n * C * D;
  w.dU = w.U + n * C * D;
  w.dY = w.dU + n * C * D;
  return w;
}

// A single LDS store that the compiler keeps as written: the pass that pairs
// LDS stores into ds_write2_b32 has emitted a wrong offset for a pair of
// accumulator-tile stores 16 columns apart (the first store landed 12 columns
// short), so the tile stores of the grads kernel go through this.
typedef __attribute__((address_space(3))) float lds_f32;
__device__ __forceinline__ void st_lds(float* p, float v) { *(volatile lds_f32*)p = v; }

// Wave index as a wave-uniform (scalar) value, so loops and branches on it
// are scalar and never exec-masked.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
}

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Sum over the 16 lanes of a DPP row (every lane of the row receives it).
__device__ __forceinline__ float row16_sum(float x) {
  auto mv = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, v), decltype(ctrl)::value,
                                         0xF, 0xF, false));
  };
  x += mv(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
  x += mv(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
  x += mv(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  x += mv(x, std::integral_constant<int, 0x140>{});  // row_mirror
  return x;
}

__device__ __forceinline__ size_t tok_off(int b, int t, int h, int T, int H) {
  return (((size_t)b * T + t) * H + h) * D;
}

// Rows t0 .. t0 + C - 1 of a [B, T, H, D] tensor into an LDS tile [C][ld]
// of type TL (zeros past T), 256 threads.
template <class TIn, class TL>
__device__ __forceinline__ void load_tile(TL* dst, int ld, const TIn* src, int b, int t0, int h,
                                          int T, int H) {
  typedef typename Vec16<TIn>::type vec;
  constexpr int VN = Vec16<TIn>::N;
  constexpr int VPR = D / VN;
  for (int i = threadIdx.x; i < C * VPR; i += 256) {
    const int r = i / VPR, cv = i % VPR;
    const int t = t0 + r;
    vec x;
    if (t < T) {
      x = *reinterpret_cast<const vec*>(src + (((size_t)b * T + t) * H + h) * D + cv * VN);
    } else {
#pragma unroll
      for (int e = 0; e < VN; ++e) x[e] = from_f32<TIn>(0.f);
    }
#pragma unroll
    for (int e = 0; e < VN; ++e) dst[r * ld + cv * VN + e] = from_f32<TL>(to_f32(x[e]));
  }
}

// ---------------------------------------------------------------------------
// prep: per-chunk gates, Gram matrices, triangular inverse (f32 record).
// ---------------------------------------------------------------------------
template <class TIn>
__global__ __launch_bounds__(256) void bwdc_prep_kernel(const TIn* __restrict__ q,
                                                        const TIn* __restrict__ k,
                                                        const float* __restrict__ alpha,
                                                        const float* __restrict__ beta, int T,
                                                        int H, int NC, float scale,
                                                        float* __restrict__ rec_all) {
  typedef Mfma<TIn> M;
  constexpr int LK = D + Vec16<TIn>::N;
  // The A matrix and the block-substitution scratch reuse the Q and K tiles'
  // LDS once the Gram products are in registers (35 KB per work-group with
  // bf16 inputs, so four work-groups share a CU).
  __shared__ __align__(16) TIn Ks[C * LK];
  __shared__ __align__(16) TIn Qs[C * LK];
  __shared__ float gam[C], bet[C];
  static_assert(sizeof(TIn) * C * LK >= sizeof(float) * C * LC, "A fits in the Q tile");
  static_assert(sizeof(TIn) * C * LK >= sizeof(float) * 4 * 16 * 16, "scratch fits in the K tile");
  float* Am = reinterpret_cast<float*>(Qs);
  float (*Xs)[16 * 16] = reinterpret_cast<float (*)[16 * 16]>(Ks);

  const int tid = threadIdx.x, wave = tid >> 6, l = lane_id();
  const int chunk = blockIdx.x % NC, bh = blockIdx.x / NC;
  const int b = bh / H, h = bh % H, t0 = chunk * C;
  float* rec = rec_all + (size_t)blockIdx.x * REC;

  if (wave == 0) {
    float la = 0.f, bt = 0.f;
    if (t0 + l < T) {
      const size_t gi = ((size_t)b * T + t0 + l) * H + h;
      la = logf(alpha[gi]);
      bt = beta[gi];
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(la, off);
      if (l >= off) la += y;
    }
    gam[l] = la;
    bet[l] = bt;
    rec[3 * C * C + l] = la;
  }
  load_tile(Ks, LK, k, b, t0, h, T, H);
  load_tile(Qs, LK, q, b, t0, h, T, H);
  __syncthreads();

  // Lower block triangle of K K^T (x < 10) and Q K^T (x >= 10): 20 tiles.
  float* Pg = rec + C * C;
  float* Gg = rec + 2 * C * C;
  f32x4 accs[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int x = wave + 4 * j;
    const int which = x / 10, y = x % 10;
    const int ti = y < 1 ? 0 : y < 3 ? 1 : y < 6 ? 2 : 3;
    const int tj = y - ti * (ti + 1) / 2;
    const TIn* Arow = (which ? Qs : Ks) + ti * 16 * LK;
    const TIn* Brow = Ks + tj * 16 * LK;
    accs[j] = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += M::KSTEP)
      accs[j] = M::mma(frag_k(Arow, LK, k0, D), frag_k(Brow, LK, k0, D), accs[j]);
  }
  __syncthreads();  // K and Q tiles no longer read: their LDS takes A and the scratch
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int x = wave + 4 * j;
    const int which = x / 10, y = x % 10;
    const int ti = y < 1 ? 0 : y < 3 ? 1 : y < 6 ? 2 : 3;
    const int tj = y - ti * (ti + 1) / 2;
    const f32x4 acc = accs[j];
    const int col = tj * 16 + (l & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ti * 16 + 4 * (l >> 4) + i;
      const float gr = __expf(gam[r] - gam[col]);
      if (which == 0) {
        Am[r * LC + col] = col < r ? bet[r] * gr * acc[i] : 0.f;
        Gg[r * C + col] = col < r ? acc[i] : 0.f;
      } else {
        Pg[r * C + col] = col <= r ? scale * gr * acc[i] : 0.f;
      }
    }
  }
  // Blocks above the diagonal of the record's P and Gk.
  for (int i = tid; i < C * C; i += 256) {
    const int r = i / C, c = i % C;
    if ((c >> 4) > (r >> 4)) {
      Pg[i] = 0.f;
      Gg[i] = 0.f;
      Am[r * LC + c] = 0.f;
    }
  }
  __syncthreads();

  // Tm = (I + A)^-1 in place: diagonal blocks by forward substitution (lane
  // = (block, column)), then block rows I = 1..3: T_IJ = -T_II sum_K A_IK T_KJ.
  if (wave == 0) {
    const int d0 = (l >> 4) * 16, j = l & 15;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) s -= Am[(d0 + r) * LC + d0 + i] * t[i];
      t[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Am[(d0 + r) * LC + d0 + j] = t[r];
  }
  __syncthreads();
  for (int I = 1; I < 4; ++I) {
    const int J = wave;
    f32x4 x = zero4();
    if (J < I) {
      for (int K = J; K < I; ++K) {
        const float* Ab = Am + (I * 16) * LC + K * 16;
        const float* Tb = Am + (K * 16) * LC + J * 16;
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4)
          x = mma4(Ab[(l & 15) * LC + k0 + (l >> 4)], Tb[(k0 + (l >> 4)) * LC + (l & 15)], x);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Xs[J][(4 * (l >> 4) + i) * 16 + (l & 15)] = x[i];
    }
    __syncthreads();
    if (J < I) {
      f32x4 y = zero4();
      const float* Tii = Am + (I * 16) * LC + I * 16;
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4)
        y = mma4(Tii[(l & 15) * LC + k0 + (l >> 4)], Xs[J][(k0 + (l >> 4)) * 16 + (l & 15)], y);
#pragma unroll
      for (int i = 0; i < 4; ++i) Am[(I * 16 + 4 * (l >> 4) + i) * LC + J * 16 + (l & 15)] = -y[i];
    }
    __syncthreads();
  }
  for (int i = tid; i < C * C / 4; i += 256) {
    const int r = i / (C / 4), c4 = i % (C / 4);
    *reinterpret_cast<f32x4*>(rec + r * C + c4 * 4) =
        *reinterpret_cast<const f32x4*>(Am + r * LC + c4 * 4);
  }
}

// Per-chunk gate vectors from the record's gam: g, d, and g_{C-1}.
struct Gates {
  float g[C], d[C], bet[C], gC;
};
__device__ __forceinline__ void load_gates(Gates& gs, const float* rec, const float* beta, int b,
                                           int t0, int h, int T, int H) {
  const int tid = threadIdx.x;
  if (tid < C) {
    const float gm = rec[3 * C * C + tid];
    const float gl = rec[3 * C * C + C - 1];
    gs.g[tid] = __expf(gm);
    gs.d[tid] = __expf(gl - gm);
    gs.bet[tid] = (t0 + tid < T) ? beta[((size_t)b * T + t0 + tid) * H + h] : 0.f;
    if (tid == 0) gs.gC = __expf(gl);
  }
}

// Per-chunk inputs of the sequential kernels, one chunk ahead in registers
// (512 threads): K (and Q) tiles in the input type, the record's Tm (and P),
// the gates' log cumsum and beta (threads 0..63).
template <class TIn>
struct TileRegs {
  typedef typename Vec16<TIn>::type vec;
  static constexpr int VN = Vec16<TIn>::N;
  static constexpr int KV = C * D / VN / 512;  // K-tile vectors per thread
  vec x[KV];
  __device__ __forceinline__ void issue(const TIn* src, int b, int t0, int h, int T, int H) {
#pragma unroll
    for (int u = 0; u < KV; ++u) {
      const int i = threadIdx.x + 512 * u, r = i / (D / VN), cv = i % (D / VN);
      if (t0 + r < T) {
        x[u] = *reinterpret_cast<const vec*>(src + tok_off(b, t0 + r, h, T, H) + cv * VN);
      } else {
#pragma unroll
        for (int e = 0; e < VN; ++e) x[u][e] = from_f32<TIn>(0.f);
      }
    }
  }
  __device__ __forceinline__ void store(TIn* dst, int ld) const {
#pragma unroll
    for (int u = 0; u < KV; ++u) {
      const int i = threadIdx.x + 512 * u, r = i / (D / VN), cv = i % (D / VN);
      *reinterpret_cast<vec*>(dst + r * ld + cv * VN) = x[u];
    }
  }
  // Unconditional loads (rows past T read row T - 1; store_f32_rows zeroes
  // them): with no load under a branch the compiler does not wait for the
  // loads at the branch's end, so they stay in flight.
  __device__ __forceinline__ void issue_clamped(const TIn* src, int b, int t0, int h, int T,
                                                int H) {
#pragma unroll
    for (int u = 0; u < KV; ++u) {
      const int i = threadIdx.x + 512 * u, r = i / (D / VN), cv = i % (D / VN);
      x[u] = *reinterpret_cast<const vec*>(src + tok_off(b, min(t0 + r, T - 1), h, T, H) + cv * VN);
    }
  }
  __device__ __forceinline__ void store_f32_rows(float* dst, int ld, int t0, int T) const {
#pragma unroll
    for (int u = 0; u < KV; ++u) {
      const int i = threadIdx.x + 512 * u, r = i / (D / VN), cv = i % (D / VN);
      const bool in = t0 + r < T;
#pragma unroll
      for (int e = 0; e < VN; e += 4)
        *reinterpret_cast<f32x4*>(dst + r * ld + cv * VN + e) =
            in ? f32x4{to_f32(x[u][e]), to_f32(x[u][e + 1]), to_f32(x[u][e + 2]),
                       to_f32(x[u][e + 3])}
               : zero4();
    }
  }
};
// A C x C f32 record matrix: 2 vectors per thread.
struct RecRegs {
  f32x4 x[2];
  __device__ __forceinline__ void issue(const float* src) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + 512 * u;
      x[u] = *reinterpret_cast<const f32x4*>(src + (i >> 4) * C + (i & 15) * 4);
    }
  }
  __device__ __forceinline__ void store(float* dst) const {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + 512 * u;
      *reinterpret_cast<f32x4*>(dst + (i >> 4) * LC + (i & 15) * 4) = x[u];
    }
  }
};
struct GateRegs {
  float gm = 0.f, bt = 0.f;
  __device__ __forceinline__ void issue(const float* rec, const float* beta, int b, int t0, int h,
                                        int T, int H) {
    const int tid = threadIdx.x;
    if (tid < C) {
      gm = rec[3 * C * C + tid];
      bt = (t0 + tid < T) ? beta[((size_t)b * T + t0 + tid) * H + h] : 0.f;
    }
  }
  // Threads 0..63 are wave 0: the last row's log gate by a lane broadcast.
  __device__ __forceinline__ void store(Gates& gs) const {
    const int tid = threadIdx.x;
    if (tid < C) {
      const float gl = __shfl(gm, C - 1);
      gs.g[tid] = __expf(gm);
      gs.d[tid] = __expf(gl - gm);
      gs.bet[tid] = bt;
      if (tid == 0) gs.gC = __expf(gl);
    }
  }
};

// ---------------------------------------------------------------------------
// forward: S entering every chunk, Vm and U (value slice of DVS columns).
// Wave w (8 waves): state key rows 16 w .. 16 w + 15; token rows 16 (w >> 1)
// .. + 15 and column tiles (w & 1) NT / 2 + {0 .. NT / 2 - 1} of the C x DVS
// products.
// ---------------------------------------------------------------------------
template <class TIn, int DVS>
__global__ __launch_bounds__(512) void bwdc_fwd_kernel(const TIn* __restrict__ k,
                                                       const TIn* __restrict__ v,
                                                       const float* __restrict__ beta,
                                                       const float* __restrict__ state_in, int T,
                                                       int H, int NC, int NS, float* __restrict__ wsb) {
  constexpr int NT = DVS / 16, NH = NT / 2;
  constexpr int LK = D + 8;        // K tile stride (input type)
  constexpr int LS = DVS + 16;     // [rows][DVS] tiles read m-contiguous
  __shared__ __align__(16) TIn Ks[C * LK];
  __shared__ __align__(16) float Ts[C * LC];
  __shared__ __align__(16) float Ss[D * LS];
  __shared__ __align__(16) float Ys[C * LS];
  __shared__ __align__(16) float Us[C * LS];
  __shared__ Gates gs;

  const int w = wave_index(), l = lane_id();
  int bh, slice;
  xcd_group_map(blockIdx.x, gridDim.x / NS, NS, &bh, &slice);
  const int b = bh / H, h = bh % H, col0 = slice * DVS;
  const int rt = w >> 1, ct0 = (w & 1) * NH;
  const Ws ws = ws_split(wsb, (size_t)gridDim.x / NS * NC);

  f32x4 S[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    S[n] = zero4();
    if (state_in) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[n][i] = state_in[((size_t)bh * D + 16 * w + 4 * (l >> 4) + i) * D + col0 + n * 16 +
                           (l & 15)];
    }
  }

  TileRegs<TIn> kr;
  RecRegs tr;
  GateRegs gr;
  uint32_t vr[NH][4];
  auto issue = [&](int c) {
    const int t0 = c * C;
    const float* rec = ws.rec + ((size_t)bh * NC + c) * REC;
    kr.issue(k, b, t0, h, T, H);
    tr.issue(rec);
    gr.issue(rec, beta, b, t0, h, T, H);
#pragma unroll
    for (int n = 0; n < NH; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * rt + 4 * (l >> 4) + i;
        vr[n][i] = t < T ? load_raw32(v + tok_off(b, t, h, T, H) + col0 + (ct0 + n) * 16 +
                                      (l & 15))
                         : 0u;
      }
  };
  if (NC > 0) issue(0);

  for (int c = 0; c < NC; ++c) {
    const size_t ch = (size_t)bh * NC + c;
    __syncthreads();  // the previous chunk's readers are done with LDS
    kr.store(Ks, LK);
    tr.store(Ts);
    gr.store(gs);
    float vv[NH][4];
#pragma unroll
    for (int n = 0; n < NH; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[n][i] = raw32_to_f32<TIn>(vr[n][i]);
    float* Sg = ws.S + ch * D * D;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * (l >> 4) + i, cc = n * 16 + (l & 15);
        Ss[r * LS + cc] = S[n][i];
        Sg[r * D + col0 + cc] = S[n][i];
      }
    __syncthreads();
    if (c + 1 < NC) issue(c + 1);

    // X = K S -> Vm = V - g X, Y = beta Vm.
    f32x4 X[NH];
#pragma unroll
    for (int n = 0; n < NH; ++n) X[n] = zero4();
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
      const int kk = k0 + (l >> 4);
      const float a = to_f32(Ks[(16 * rt + (l & 15)) * LK + kk]);
#pragma unroll
      for (int n = 0; n < NH; ++n)
        X[n] = mma4(a, Ss[kk * LS + (ct0 + n) * 16 + (l & 15)], X[n]);
    }
    float* Vg = ws.Vm + ch * C * D;
#pragma unroll
    for (int n = 0; n < NH; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * (l >> 4) + i, cc = (ct0 + n) * 16 + (l & 15);
        const float vm = vv[n][i] - gs.g[r] * X[n][i];
        Vg[r * D + col0 + cc] = vm;
        Ys[r * LS + cc] = gs.bet[r] * vm;
      }
    __syncthreads();

    // U = Tm Y (Tm lower triangular: tokens i < 16 (rt + 1)).
    f32x4 Uc[NH];
#pragma unroll
    for (int n = 0; n < NH; ++n) Uc[n] = zero4();
    for (int k0 = 0; k0 < 16 * (rt + 1); k0 += 4) {
      const int kk = k0 + (l >> 4);
      const float a = Ts[(16 * rt + (l & 15)) * LC + kk];
#pragma unroll
      for (int n = 0; n < NH; ++n)
        Uc[n] = mma4(a, Ys[kk * LS + (ct0 + n) * 16 + (l & 15)], Uc[n]);
    }
    float* Ug = ws.U + ch * C * D;
#pragma unroll
    for (int n = 0; n < NH; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * (l >> 4) + i, cc = (ct0 + n) * 16 + (l & 15);
        Ug[r * D + col0 + cc] = Uc[n][i];
        Us[r * LS + cc] = gs.d[r] * Uc[n][i];
      }
    __syncthreads();

    // S <- g_{C-1} S + K^T diag(d) U (key tile w).
    const float gC = gs.gC;
#pragma unroll
    for (int n = 0; n < NT; ++n) S[n] *= gC;
#pragma unroll 4
    for (int k0 = 0; k0 < C; k0 += 4) {
      const int kk = k0 + (l >> 4);
      const float a = to_f32(Ks[kk * LK + 16 * w + (l & 15)]);
#pragma unroll
      for (int n = 0; n < NT; ++n) S[n] = mma4(a, Us[kk * LS + n * 16 + (l & 15)], S[n]);
    }
  }
}

// ---------------------------------------------------------------------------
// dstate: the gradient of the state, chunks in reverse (value slice).  Wave
// w: gradient key rows 16 w .. 16 w + 15; token rows 16 (w >> 1) .. + 15 and
// column tiles (w & 1) NT / 2 + {0 .. NT / 2 - 1} of dU, dY.
// ---------------------------------------------------------------------------
template <class TIn, int DVS>
__global__ __launch_bounds__(512) void bwdc_dstate_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ beta,
    const float* __restrict__ dout, const float* __restrict__ dstate_out, float* __restrict__ dv,
    float* __restrict__ dstate_in, int T, int H, int NC, int NS, float scale,
    float* __restrict__ wsb) {
  constexpr int NT = DVS / 16, NH = NT / 2;
  constexpr int LK = D + 8;
  constexpr int LS = DVS + 16;
  constexpr int LX = DVS + 4;
  constexpr int OV = C * DVS / 4 / 512;  // dO vectors per thread
  static_assert(LX <= LC, "dX fits in the P tile");
  static_assert(OV >= 1, "dO slice covers the work-group");
  __shared__ __align__(16) TIn Ks[C * LK];
  __shared__ __align__(16) TIn Qs[C * LK];
  __shared__ __align__(16) float Ts[C * LC];
  __shared__ __align__(16) float Ps[C * LC];   // P, then dX ([token][column], stride LX)
  __shared__ __align__(16) float dOs[C * LS];
  __shared__ __align__(16) float dSs[D * LS];
  __shared__ __align__(16) float dUs[C * LS];
  __shared__ Gates gs;

  const int tid = threadIdx.x, w = wave_index(), l = lane_id();
  int bh, slice;
  xcd_group_map(blockIdx.x, gridDim.x / NS, NS, &bh, &slice);
  const int b = bh / H, h = bh % H, col0 = slice * DVS;
  const int rt = w >> 1, ct0 = (w & 1) * NH;
  const Ws ws = ws_split(wsb, (size_t)gridDim.x / NS * NC);
  float* dXs = Ps;

  f32x4 G[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    G[n] = zero4();
    if (dstate_out) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        G[n][i] = dstate_out[((size_t)bh * D + 16 * w + 4 * (l >> 4) + i) * D + col0 + n * 16 +
                             (l & 15)];
    }
  }

  TileRegs<TIn> kr, qr;
  RecRegs tr, pr;
  GateRegs gr;
  f32x4 orr[OV];
  auto issue = [&](int c) {
    const int t0 = c * C;
    const float* rec = ws.rec + ((size_t)bh * NC + c) * REC;
    kr.issue(k, b, t0, h, T, H);
    qr.issue(q, b, t0, h, T, H);
    tr.issue(rec);
    pr.issue(rec + C * C);
    gr.issue(rec, beta, b, t0, h, T, H);
#pragma unroll
    for (int u = 0; u < OV; ++u) {
      const int i = tid + 512 * u, r = i / (DVS / 4), c4 = i % (DVS / 4);
      orr[u] = zero4();
      if (t0 + r < T)
        orr[u] = *reinterpret_cast<const f32x4*>(dout + tok_off(b, t0 + r, h, T, H) + col0 +
                                                 c4 * 4);
    }
  };
  if (NC > 0) issue(NC - 1);

  for (int c = NC - 1; c >= 0; --c) {
    const int t0 = c * C;
    const size_t ch = (size_t)bh * NC + c;
    __syncthreads();
    kr.store(Ks, LK);
    qr.store(Qs, LK);
    tr.store(Ts);
    pr.store(Ps);
    gr.store(gs);
#pragma unroll
    for (int u = 0; u < OV; ++u) {
      const int i = tid + 512 * u, r = i / (DVS / 4), c4 = i % (DVS / 4);
      *reinterpret_cast<f32x4*>(dOs + r * LS + c4 * 4) = orr[u];
    }
    float* dSg = ws.dS + ch * D * D;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * (l >> 4) + i, cc = n * 16 + (l & 15);
        dSs[r * LS + cc] = G[n][i];
        dSg[r * D + col0 + cc] = G[n][i];
      }
    __syncthreads();
    if (c > 0) issue(c - 1);

    // dU = P^T dO + diag(d) K dSn   (P^T: tokens r >= 16 rt).
    f32x4 du[NH], kd[NH];
#pragma unroll
    for (int n = 0; n < NH; ++n) du[n] = kd[n] = zero4();
    for (int k0 = 16 * rt; k0 < C; k0 += 4) {
      const int kk = k0 + (l >> 4);
      const float a = Ps[kk * LC + 16 * rt + (l & 15)];
#pragma unroll
      for (int n = 0; n < NH; ++n)
        du[n] = mma4(a, dOs[kk * LS + (ct0 + n) * 16 + (l & 15)], du[n]);
    }
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
      const int kk = k0 + (l >> 4);
      const float a = to_f32(Ks[(16 * rt + (l & 15)) * LK + kk]);
#pragma unroll
      for (int n = 0; n < NH; ++n)
        kd[n] = mma4(a, dSs[kk * LS + (ct0 + n) * 16 + (l & 15)], kd[n]);
    }
    float* dUg = ws.dU + ch * C * D;
#pragma unroll
    for (int n = 0; n < NH; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * (l >> 4) + i, cc = (ct0 + n) * 16 + (l & 15);
        const float x = du[n][i] + gs.d[r] * kd[n][i];
        dUg[r * D + col0 + cc] = x;
        dUs[r * LS + cc] = x;
      }
    __syncthreads();

    // dY = Tm^T dU; dv = beta dY; dX = -beta g dY (into the P tile).
    f32x4 dy[NH];
#pragma unroll
    for (int n = 0; n < NH; ++n) dy[n] = zero4();
    for (int k0 = 16 * rt; k0 < C; k0 += 4) {
      const int kk = k0 + (l >> 4);
      const float a = Ts[kk * LC + 16 * rt + (l & 15)];
#pragma unroll
      for (int n = 0; n < NH; ++n)
        dy[n] = mma4(a, dUs[kk * LS + (ct0 + n) * 16 + (l & 15)], dy[n]);
    }
    float* dYg = ws.dY + ch * C * D;
#pragma unroll
    for (int n = 0; n < NH; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * (l >> 4) + i, cc = (ct0 + n) * 16 + (l & 15);
        const int t = t0 + r;
        dYg[r * D + col0 + cc] = dy[n][i];
        if (t < T) dv[tok_off(b, t, h, T, H) + col0 + cc] = gs.bet[r] * dy[n][i];
        dXs[r * LX + cc] = -gs.bet[r] * gs.g[r] * dy[n][i];
      }
    __syncthreads();

    // dS <- g_{C-1} dS + Q^T diag(scale g) dO + K^T dX (key tile w).
    const float gC = gs.gC;
#pragma unroll
    for (int n = 0; n < NT; ++n) G[n] *= gC;
#pragma unroll 2
    for (int k0 = 0; k0 < C; k0 += 4) {
      const int kk = k0 + (l >> 4);
      const float aq = scale * gs.g[kk] * to_f32(Qs[kk * LK + 16 * w + (l & 15)]);
      const float ak = to_f32(Ks[kk * LK + 16 * w + (l & 15)]);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const float bo = dOs[kk * LS + n * 16 + (l & 15)];
        const float bx = dXs[kk * LX + n * 16 + (l & 15)];
        G[n] = mma4(ak, bx, mma4(aq, bo, G[n]));
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dstate_in[((size_t)bh * D + 16 * w + 4 * (l >> 4) + i) * D + col0 + n * 16 + (l & 15)] =
          G[n][i];
}

// ---------------------------------------------------------------------------
// grads: dq, dk, dalpha, dbeta of one chunk.
// ---------------------------------------------------------------------------
// LDS of the value passes (32 columns of S, dSn, dO, dY, U, Vm, dU).
struct GradV {
  float S[D * (QV + 4)], dS[D * (QV + 4)];
  float dO[C * (QV + 4)], dY[C * (QV + 4)], U[C * (QV + 4)], Vm[C * (QV + 4)], dU[C * (QV + 4)];
};
// LDS of the key-side part.
struct GradK {
  float K[C * (D + 4)], Q[C * (D + 4)];
  float Tm[C * LC], dT[C * LC], M1[C * LC], Ep[C * LC];
};
constexpr int LV = QV + 4;
constexpr int LKF = D + 4;

// Lower block-triangle tile y (0..9) of a C x C matrix: row tile, column tile.
__device__ __forceinline__ int low_rt(int y) { return (y >= 1) + (y >= 3) + (y >= 6); }
__device__ __forceinline__ int low_ct(int y) {
  const int rt = low_rt(y);
  return y - rt * (rt + 1) / 2;
}

// The value passes' inputs (32 columns of S, dSn, dO, dY, U, Vm, dU), one
// pass ahead in registers: 9 16-byte pieces per thread (512 threads).
struct PassRegs {
  f32x4 x[9];
};
__device__ __forceinline__ void pass_issue(PassRegs& pr, const Ws& ws, size_t ch, const float* dout,
                                           int b, int t0, int h, int T, int H, int c0) {
  const int tid = threadIdx.x;
  const float* S = ws.S + ch * D * D + c0;
  const float* dS = ws.dS + ch * D * D + c0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = tid + 512 * u, r = i >> 3, c4 = i & 7;
    pr.x[u] = *reinterpret_cast<const f32x4*>(S + r * D + c4 * 4);
    pr.x[2 + u] = *reinterpret_cast<const f32x4*>(dS + r * D + c4 * 4);
  }
  const int r = tid >> 3, c4 = tid & 7;
  // (unconditional: rows past T read row T - 1 and are zeroed in pass_store)
  pr.x[4] = *reinterpret_cast<const f32x4*>(dout + tok_off(b, min(t0 + r, T - 1), h, T, H) + c0 +
                                            c4 * 4);
  const size_t o = ch * C * D + r * D + c0 + c4 * 4;
  pr.x[5] = *reinterpret_cast<const f32x4*>(ws.dY + o);
  pr.x[6] = *reinterpret_cast<const f32x4*>(ws.U + o);
  pr.x[7] = *reinterpret_cast<const f32x4*>(ws.Vm + o);
  pr.x[8] = *reinterpret_cast<const f32x4*>(ws.dU + o);
}
__device__ __forceinline__ void pass_store(const PassRegs& pr, GradV& sv, int t0, int T) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = tid + 512 * u, r = i >> 3, c4 = i & 7;
    *reinterpret_cast<f32x4*>(sv.S + r * LV + c4 * 4) = pr.x[u];
    *reinterpret_cast<f32x4*>(sv.dS + r * LV + c4 * 4) = pr.x[2 + u];
  }
  const int o = (tid >> 3) * LV + (tid & 7) * 4;
  *reinterpret_cast<f32x4*>(sv.dO + o) = t0 + (tid >> 3) < T ? pr.x[4] : zero4();
  *reinterpret_cast<f32x4*>(sv.dY + o) = pr.x[5];
  *reinterpret_cast<f32x4*>(sv.U + o) = pr.x[6];
  *reinterpret_cast<f32x4*>(sv.Vm + o) = pr.x[7];
  *reinterpret_cast<f32x4*>(sv.dU + o) = pr.x[8];
}

// Work of wave w (8 waves): token tiles 2 (w & 1) + {0, 1} x key tiles
// 2 (w >> 1) + {0, 1} of dq_S, Z1 = dX S^T and Z2 = diag(d) U dSn^T (then dq
// and dk); lower tiles y = w and w + 8 (w < 2) of dP and of dA; lower tiles
// y = (w + 6) % 8 and that + 8 (< 10) of dTm.
template <class TIn>
__global__ __launch_bounds__(512) void bwdc_grad_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* __restrict__ dout, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dalpha, float* __restrict__ dbeta, int T, int H,
    int NC, float scale, float* __restrict__ wsb) {
  __shared__ __align__(16) char smem[sizeof(GradV) > sizeof(GradK) ? sizeof(GradV)
                                                                    : sizeof(GradK)];
  __shared__ Gates gs;
  __shared__ float gam[C], red[4][C], redz[4][C], dbY[C], dgam[C], dbA[C], colF[C], zrow[C],
      wsum[8];
  GradV& sv = *reinterpret_cast<GradV*>(smem);
  GradK& sk = *reinterpret_cast<GradK*>(smem);

  const int tid = threadIdx.x, w = wave_index(), l = lane_id();
  const int chunk = blockIdx.x % NC, bh = blockIdx.x / NC;
  const int b = bh / H, h = bh % H, t0 = chunk * C;
  const size_t ch = blockIdx.x;
  const Ws ws = ws_split(wsb, (size_t)gridDim.x);
  const float* rec = ws.rec + ch * REC;
  load_gates(gs, rec, beta, b, t0, h, T, H);
  if (tid < C) gam[tid] = rec[3 * C * C + tid];

  const int tr0 = 2 * (w & 1), kt0 = 2 * (w >> 1);
  const int nP = w < 2 ? 2 : 1;
  const int yT0 = (w + 6) & 7, nT = yT0 + 8 < 10 ? 2 : 1;
  f32x4 aQ[2][2], aZ1[2][2], aZ2[2][2], aP[2], aT[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    aP[t] = aT[t] = zero4();
#pragma unroll
    for (int m = 0; m < 2; ++m) aQ[t][m] = aZ1[t][m] = aZ2[t][m] = zero4();
  }
  float dbY_acc = 0.f, dgc_acc = 0.f;

  PassRegs pr;
  TileRegs<TIn> kx, qx;  // K and Q of the chunk, loaded during the last pass
  RecRegs tx;            // Tm, likewise
  float pv[2][4], gv[2][4];
  pass_issue(pr, ws, ch, dout, b, t0, h, T, H, 0);
  __syncthreads();  // gates in LDS
  // Per-row factors of this wave's A fragments (token rows 16 (tr0 + t) + l % 16).
  float fo[2], fy[2], fu[2], fb[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tok = (tr0 + t) * 16 + (l & 15);
    fo[t] = scale * gs.g[tok];
    fy[t] = -gs.bet[tok] * gs.g[tok];
    fu[t] = gs.d[tok];
    fb[t] = t < nT ? gs.bet[16 * low_ct(yT0 + 8 * t) + (l & 15)] : 0.f;
  }
  for (int pass = 0; pass < D / QV; ++pass) {
    if (pass) __syncthreads();  // the previous pass's readers are done
    pass_store(pr, sv, t0, T);
    __syncthreads();
    if (pass + 1 < D / QV) {
      pass_issue(pr, ws, ch, dout, b, t0, h, T, H, (pass + 1) * QV);
    } else {
      kx.issue_clamped(k, b, t0, h, T, H);
      qx.issue_clamped(q, b, t0, h, T, H);
      tx.issue(rec);
    }

    // dY . Vm per row (thread: row tid / 8, 4 columns) and <dSn, S>.
    {
      const int r = tid >> 3, cb = (tid & 7) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) dbY_acc += sv.dY[r * LV + cb + e] * sv.Vm[r * LV + cb + e];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = tid * 8 + e, rr = i / QV, cc = i % QV;
        dgc_acc += sv.dS[rr * LV + cc] * sv.S[rr * LV + cc];
      }
    }

#pragma unroll 2
    for (int k0 = 0; k0 < QV; k0 += 4) {
      const int kk = k0 + (l >> 4);
      float bS[2], bD[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int key = (kt0 + m) * 16 + (l & 15);
        bS[m] = sv.S[key * LV + kk];
        bD[m] = sv.dS[key * LV + kk];
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int tok = (tr0 + t) * 16 + (l & 15);
        const float ao = fo[t] * sv.dO[tok * LV + kk];
        const float ay = fy[t] * sv.dY[tok * LV + kk];
        const float au = fu[t] * sv.U[tok * LV + kk];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          aQ[t][m] = mma4(ao, bS[m], aQ[t][m]);
          aZ1[t][m] = mma4(ay, bS[m], aZ1[t][m]);
          aZ2[t][m] = mma4(au, bD[m], aZ2[t][m]);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (t < nP) {
          const int y = w + 8 * t;
          const float a = sv.dO[(16 * low_rt(y) + (l & 15)) * LV + kk];
          aP[t] = mma4(a, sv.U[(16 * low_ct(y) + (l & 15)) * LV + kk], aP[t]);
        }
        if (t < nT) {
          const int y = yT0 + 8 * t;
          const int i = 16 * low_ct(y) + (l & 15);
          const float a = sv.dU[(16 * low_rt(y) + (l & 15)) * LV + kk];
          aT[t] = mma4(a, fb[t] * sv.Vm[i * LV + kk], aT[t]);
        }
      }
    }
  }
  // Row sums of dY . Vm over the 8 threads of a row; <dSn, S> over the block.
  dbY_acc += __shfl_xor(dbY_acc, 1);
  dbY_acc += __shfl_xor(dbY_acc, 2);
  dbY_acc += __shfl_xor(dbY_acc, 4);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dgc_acc += __shfl_xor(dgc_acc, off);
  if (l == 0) wsum[w] = dgc_acc;
  __syncthreads();  // value passes done: the LDS becomes the key-side tiles
  if ((tid & 7) == 0) dbY[tid >> 3] = dbY_acc;

  kx.store_f32_rows(sk.K, LKF, t0, T);
  qx.store_f32_rows(sk.Q, LKF, t0, T);
  tx.store(sk.Tm);
  // P and K K^T on this wave's dA / dP tiles (used at the dA stage below).
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int y = w + 8 * (t < nP ? t : 0);
      const int o = (16 * low_rt(y) + 4 * (l >> 4) + i) * C + 16 * low_ct(y) + (l & 15);
      pv[t][i] = rec[C * C + o];
      gv[t][i] = rec[2 * C * C + o];
    }
  // dTm, strictly lower part (the only part that reaches dA); zeros above.
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t >= nT) continue;
    const int y = yT0 + 8 * t;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * low_rt(y) + 4 * (l >> 4) + i, cc = 16 * low_ct(y) + (l & 15);
      st_lds(&sk.dT[r * LC + cc], cc < r ? aT[t][i] : 0.f);
    }
  }
  for (int i = tid; i < C * C; i += 512) {
    const int r = i / C, cc = i % C;
    if ((cc >> 4) > (r >> 4)) sk.dT[r * LC + cc] = 0.f;
  }
  __syncthreads();

  // rho: dq_S.q + Z1.k - Z2.k per row, and Z2.k (key-group partials).
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 16 * (tr0 + t) + 4 * (l >> 4) + i;
      float sq = 0.f, z = 0.f;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int key = (kt0 + m) * 16 + (l & 15);
        const float kv = sk.K[tok * LKF + key];
        sq += aQ[t][m][i] * sk.Q[tok * LKF + key] + aZ1[t][m][i] * kv;
        z += aZ2[t][m][i] * kv;
      }
      sq = row16_sum(sq);
      z = row16_sum(z);
      if ((l & 15) == 0) {
        red[w >> 1][tok] = sq - z;
        redz[w >> 1][tok] = z;
      }
    }
  }

  // M1 = dTm Tm^T: row tile w >> 1, column tiles 2 (w & 1) + {0, 1}
  // (contraction b < 16 min(row tile, column tile) + 16).
  {
    const int at = w >> 1;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * (w & 1) + jj;
      f32x4 m1 = zero4();
      const int kend = 16 * (min(at, j) + 1);
      for (int k0 = 0; k0 < kend; k0 += 4) {
        const int kk = k0 + (l >> 4);
        m1 = mma4(sk.dT[(16 * at + (l & 15)) * LC + kk], sk.Tm[(16 * j + (l & 15)) * LC + kk], m1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st_lds(&sk.M1[(16 * at + 4 * (l >> 4) + i) * LC + 16 * j + (l & 15)], m1[i]);
    }
  }
  __syncthreads();

  // dA = -Tm^T M1 on lower tiles y = w, w + 8 (contraction a >= 16 row tile).
  f32x4 da[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    da[t] = zero4();
    if (t >= nP) continue;
    const int y = w + 8 * t, rt = low_rt(y), ct = low_ct(y);
    for (int k0 = 16 * rt; k0 < C; k0 += 4) {
      const int kk = k0 + (l >> 4);
      da[t] = mma4(sk.Tm[kk * LC + 16 * rt + (l & 15)], sk.M1[kk * LC + 16 * ct + (l & 15)], da[t]);
    }
  }
  __syncthreads();  // Tm, dTm, M1 no longer read

  // E2 = diag(beta) (G o dA) -> dT tile; H = dA o G o Gk (row sums: dbeta's
  // A part) -> M1 tile; F = dP o P + dA o A -> Ep; E1 = scale G o dP -> Tm tile.
  float* E2s = sk.dT;
  float* Hs = sk.M1;
  float* E1s = sk.Tm;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t >= nP) continue;
    const int y = w + 8 * t, rt = low_rt(y), ct = low_ct(y);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rt + 4 * (l >> 4) + i, cc = 16 * ct + (l & 15);
      const float gr = cc <= r ? __expf(gam[r] - gam[cc]) : 0.f;
      float e2 = 0.f, hh = 0.f, e1 = 0.f, f = 0.f;
      if (cc < r) {
        const float a = -da[t][i] * gr;  // dA_ri G_ri
        hh = a * gv[t][i];
        e2 = gs.bet[r] * a;
        f = gs.bet[r] * hh;
      }
      if (cc <= r) {
        e1 = scale * gr * aP[t][i];
        f += aP[t][i] * pv[t][i];
      }
      st_lds(&E2s[r * LC + cc], e2);
      st_lds(&Hs[r * LC + cc], hh);
      st_lds(&E1s[r * LC + cc], e1);
      st_lds(&sk.Ep[r * LC + cc], f);
    }
  }
  for (int i = tid; i < C * C; i += 512) {
    const int r = i / C, cc = i % C;
    if ((cc >> 4) > (r >> 4)) {
      E2s[r * LC + cc] = 0.f;
      Hs[r * LC + cc] = 0.f;
      E1s[r * LC + cc] = 0.f;
      sk.Ep[r * LC + cc] = 0.f;
    }
  }
  __syncthreads();

  // Row sums of F and H and column sums of F, 8 threads per row / column.
  {
    const int x = tid >> 3, p0 = (tid & 7) * 8;
    float fr = 0.f, hr = 0.f, fc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      fr += sk.Ep[x * LC + p0 + e];
      hr += Hs[x * LC + p0 + e];
      fc += sk.Ep[(p0 + e) * LC + x];
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      fr += __shfl_xor(fr, off);
      hr += __shfl_xor(hr, off);
      fc += __shfl_xor(fc, off);
    }
    if ((tid & 7) == 0) {
      dgam[x] = fr + red[0][x] + red[1][x] + red[2][x] + red[3][x];
      dbA[x] = dbY[x] + hr;
      colF[x] = fc;
      zrow[x] = redz[0][x] + redz[1][x] + redz[2][x] + redz[3][x];
    }
  }

  // dq += E1 K; dk += E1^T Q + (E2 + E2^T) K.
#pragma unroll 2
  for (int k0 = 0; k0 < C; k0 += 4) {
    const int kk = k0 + (l >> 4);
    float bK[2], bQ[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int key = (kt0 + m) * 16 + (l & 15);
      bK[m] = sk.K[kk * LKF + key];
      bQ[m] = sk.Q[kk * LKF + key];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int tok = 16 * (tr0 + t) + (l & 15);
      const float a1 = E1s[tok * LC + kk];
      const float a1t = E1s[kk * LC + tok];
      const float a2 = E2s[tok * LC + kk] + E2s[kk * LC + tok];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        aQ[t][m] = mma4(a1, bK[m], aQ[t][m]);
        aZ1[t][m] = mma4(a1t, bQ[m], mma4(a2, bK[m], aZ1[t][m]));
      }
    }
  }
  __syncthreads();  // dgam, colF, dbA complete

  // dgam = row sums - column sums of F + rho (+ the last row's terms);
  // dlog(alpha) = its reverse cumulative sum; dalpha = dlog(alpha) / alpha.
  if (w == 0) {
    const int r = C - 1 - l, t = t0 + r;
    float x = dgam[r] - colF[r];
    float zs = zrow[l];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) zs += __shfl_xor(zs, off);
    if (r == C - 1) {
      float ws8 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ws8 += wsum[i];
      x += gs.gC * ws8 + zs;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (l >= off) x += y;
    }
    if (t < T) {
      const size_t gi = ((size_t)b * T + t) * H + h;
      dalpha[gi] = x / alpha[gi];
      dbeta[gi] = dbA[r];
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 16 * (tr0 + t) + 4 * (l >> 4) + i, tt = t0 + tok;
      if (tt >= T) continue;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int key = (kt0 + m) * 16 + (l & 15);
        const size_t o = tok_off(b, tt, h, T, H) + key;
        dq[o] = aQ[t][m][i];
        dk[o] = aZ1[t][m][i] + aZ2[t][m][i];
      }
    }
}

template <class TIn>
hipError_t launch_bwdc_t(const BwdArgs& p) {
  constexpr int DVS = sizeof(TIn) == 2 ? 64 : 32;
  constexpr int NS = D / DVS;
  const int NC = (p.T + C - 1) / C;
  const int BH = p.B * p.H;
  float* ws = (float*)p.workspace;
  const hipStream_t st = (hipStream_t)p.stream;
  const TIn *q = (const TIn*)p.q, *k = (const TIn*)p.k, *v = (const TIn*)p.v;
  if (NC > 0) {
    hipLaunchKernelGGL(bwdc_prep_kernel<TIn>, dim3(BH * NC), dim3(256), 0, st, q, k, p.alpha,
                       p.beta, p.T, p.H, NC, p.scale, ws_split(ws, (size_t)BH * NC).rec);
    hipLaunchKernelGGL((bwdc_fwd_kernel<TIn, DVS>), dim3(BH * NS), dim3(512), 0, st, k, v, p.beta,
                       p.state_in, p.T, p.H, NC, NS, ws);
  }
  hipLaunchKernelGGL((bwdc_dstate_kernel<TIn, DVS>), dim3(BH * NS), dim3(512), 0, st, q, k,
                     p.beta, p.dout, p.dstate_out, p.dv, p.dstate_in, p.T, p.H, NC, NS, p.scale,
                     ws);
  if (NC > 0)
    hipLaunchKernelGGL(bwdc_grad_kernel<TIn>, dim3(BH * NC), dim3(512), 0, st, q, k, p.alpha,
                       p.beta, p.dout, p.dq, p.dk, p.dalpha, p.dbeta, p.T, p.H, NC, p.scale, ws);
  return hipGetLastError();
}

}  // namespace

bool backward_chunked_supported(int Dk, int Dv) { return Dk == D && Dv == D; }

size_t backward_chunked_workspace_bytes(int B, int T, int H) {
  const size_t nc = ((size_t)T + C - 1) / C;
  return (size_t)B * H * nc * PER_CHUNK * sizeof(float);
}

hipError_t launch_backward_chunked(const BwdArgs& p) {
  return p.bf16 ? launch_bwdc_t<bf16>(p) : launch_bwdc_t<float>(p);
}

}  // namespace gdn
