// Chunk-parallel GDN prefill for gfx950.
//
// Method: "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 3.1.2, S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1}
// + beta_t k_t v_t^T, o_t = scale * S_t^T q_t, computed chunk by chunk with an
// exact algebraic rewrite (the WY/UT form the page cites for its kernels).
// Within a chunk of C tokens r = 0..C-1 entering with state S0, let
// gam_r = sum_{j<=r} log alpha_j and g_r = exp(gam_r).  One step is
// S_r = alpha_r S_{r-1} + k_r u_r^T with u_r = beta_r (v_r - alpha_r S_{r-1}^T k_r);
// unrolling gives the lower-triangular system
//   (I + A) U = diag(beta) (V - diag(g) K S0),
//   A_ri = beta_r exp(gam_r - gam_i) k_r.k_i  (i < r),
// so with Tm = (I + A)^-1:
//   U   = Tm diag(beta) (V - diag(g) (K S0))
//   O   = diag(scale g) Q S0 + Pm U,   Pm_ri = scale exp(gam_r - gam_i) q_r.k_i (i <= r)
//   S_C = g_C S0 + K^T diag(exp(gam_C - gam)) U
// Everything that does not involve S0 (gam, Tm, Pm) is per-chunk and fully
// parallel: kernel 1.  The rest is a sequential walk over chunks that carries
// S in f32 MFMA accumulators: kernel 2.  Columns of S (the value dimension)
// evolve independently, so kernel 2 splits Dv into slices of DVS columns, one
// work-group each, to put enough work-groups on the chip.
//
// This two-kernel form serves the shapes the per-head kernels
// (gdn_prefill_head.hip) do not: f32 inputs, head dimensions other than
// Dk = Dv = 128, chunks of 16 or 32 tokens.
//
// Ragged tails: the last chunk is padded with identity tokens (alpha = 1,
// beta = 0, q = k = v = 0), which leave S unchanged and read 0.
//
// Precision (bf16 inputs): the Gram products K K^T and Q K^T take the bf16
// inputs directly (bf16 MFMA, exact products, f32 accumulation).  Every
// product on the state path (K S0, Q S0, Tm Y, Pm U, K^T U) takes f16
// operands (f16 MFMA, same rate as bf16): unit-scale bf16 inputs convert to
// f16 exactly, and the intermediates S, Y, U, Tm, Pm are rounded with 3 more
// mantissa bits than bf16 would give.  Accumulation is f32 everywhere and the
// master state S is f32.  f32 inputs use f32 MFMA throughout.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

size_t prefill_record_bytes(int C, bool bf16) {
  const size_t e = bf16 ? 2 : 4;
  const size_t b = 2 * (size_t)C * C * e + (size_t)C * 4;
  return (b + 255) / 256 * 256;
}

size_t prefill_workspace_bytes(int B, int T, int H, int Dk, int Dv, int C, bool bf16) {
  PrefillArgs p{};
  p.B = B; p.T = T; p.H = H; p.Dk = Dk; p.Dv = Dv; p.chunk = C; p.bf16 = bf16;
  if (prefill_head_supported(p)) return prefill_head_workspace_bytes(B, T, H);
  const size_t nc = ((size_t)T + C - 1) / C;
  return (size_t)B * H * nc * prefill_record_bytes(C, bf16);
}

// ---------------------------------------------------------------------------
// Kernel 1: per-chunk gate cumsum, Gram products, triangular inverse.
// One work-group (4 waves) per (b, h, chunk).
// ---------------------------------------------------------------------------
template <class TIn, int C, int DK>
__global__ __launch_bounds__(256) void chunk_prep_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const float* __restrict__ alpha, const float* __restrict__ beta, int T,
    int H, int NC, float scale, char* __restrict__ ws, size_t rec_bytes) {
  typedef Mfma<TIn> M;                        // Gram products on the inputs
  typedef typename OperandOf<TIn>::type OpT;  // type of the stored Tm, Pm
  typedef typename Vec16<TIn>::type vec;
  typedef typename Vec16<OpT>::type ovec;
  static_assert(sizeof(OpT) == sizeof(TIn), "operand and input sizes differ");
  constexpr int VN = Vec16<TIn>::N;
  constexpr int PAD = VN;
  constexpr int LDK = DK + PAD;      // K/Q tile row stride (elements)
  constexpr int LDP = C + PAD;       // staged Pm row stride
  constexpr int LDA = C + 4;         // f32 A / Tm row stride
  constexpr int NB = C / 16;         // 16-row blocks per chunk
  constexpr int QREG = (C * LDK > C * LDP) ? C * LDK : C * LDP;

  __shared__ __align__(16) TIn Ks[C * LDK];
  __shared__ __align__(16) TIn Qs[QREG];  // Q tile, later the staged Pm
  __shared__ __align__(16) float Am[C * LDA];
  __shared__ __align__(16) float Xs[4][16 * 16];
  __shared__ float gam[C], bet[C];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = lane_id();
  const int chunk = blockIdx.x % NC;
  const int bh = blockIdx.x / NC;
  const int b = bh / H, h = bh % H;
  const int t0 = chunk * C;

  // 1. log gates and their inclusive cumsum over the chunk (one wave).
  if (wave == 0) {
    float la = 0.f, bt = 0.f;
    if (l < C && t0 + l < T) {
      const size_t gi = ((size_t)b * T + t0 + l) * H + h;
      la = logf(alpha[gi]);
      bt = beta[gi];
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(la, off);
      if (l >= off) la += y;
    }
    if (l < C) {
      gam[l] = la;
      bet[l] = bt;
    }
  }
  // 2. K and Q tiles of the chunk (zero rows past T).
  constexpr int VPR = DK / VN;
  for (int i = tid; i < C * VPR; i += 256) {
    const int r = i / VPR, cv = i % VPR;
    const int t = t0 + r;
    vec xk, xq;
    if (t < T) {
      const size_t off = (((size_t)b * T + t) * H + h) * DK + cv * VN;
      xk = *reinterpret_cast<const vec*>(k + off);
      xq = *reinterpret_cast<const vec*>(q + off);
    } else {
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        xk[e] = from_f32<TIn>(0.f);
        xq[e] = from_f32<TIn>(0.f);
      }
    }
    *reinterpret_cast<vec*>(Ks + r * LDK + cv * VN) = xk;
    *reinterpret_cast<vec*>(Qs + r * LDK + cv * VN) = xq;
  }
  __syncthreads();

  // 3. Gram tiles K K^T and Q K^T (lower block triangle), kept in registers.
  constexpr int NTILE = 2 * NB * NB;
  constexpr int TPW = (NTILE + 3) / 4;
  f32x4 acc[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    acc[j] = zero4();
    const int x = wave + 4 * j;
    if (x < NTILE) {
      const int which = x / (NB * NB);  // 0: K K^T, 1: Q K^T
      const int ti = (x % (NB * NB)) / NB, tj = x % NB;
      if (tj <= ti) {
        const TIn* Arow = (which ? Qs : Ks) + ti * 16 * LDK;
        const TIn* Brow = Ks + tj * 16 * LDK;
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += M::KSTEP)
          acc[j] = M::mma(frag_k(Arow, LDK, k0, DK), frag_k(Brow, LDK, k0, DK), acc[j]);
      }
    }
  }
  __syncthreads();  // Q tile no longer read: its storage takes Pm
  OpT* Ps = reinterpret_cast<OpT*>(Qs);
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int x = wave + 4 * j;
    if (x < NTILE) {
      const int which = x / (NB * NB);
      const int ti = (x % (NB * NB)) / NB, tj = x % NB;
      const int col = tj * 16 + (l & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = ti * 16 + 4 * (l >> 4) + i;
        const float d = __expf(gam[r] - gam[col]);
        if (which == 0) {
          Am[r * LDA + col] = (col < r) ? bet[r] * d * acc[j][i] : 0.f;
        } else {
          Ps[r * LDP + col] = from_f32<OpT>((col <= r) ? scale * d * acc[j][i] : 0.f);
        }
      }
    }
  }
  __syncthreads();

  // 4. Tm = (I + A)^-1, in place in Am.
  // 4a. Diagonal 16x16 blocks by forward substitution: lane = (block, column).
  if (wave == 0 && (l >> 4) < NB) {
    const int d0 = (l >> 4) * 16, j = l & 15;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) s -= Am[(d0 + r) * LDA + d0 + i] * t[i];
      t[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Am[(d0 + r) * LDA + d0 + j] = t[r];
  }
  __syncthreads();
  // 4b. Off-diagonal blocks, one block row at a time:
  //     T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ   (wave J computes block J).
  for (int I = 1; I < NB; ++I) {
    const int J = wave;
    f32x4 x = zero4();
    if (J < I) {
      for (int K = J; K < I; ++K) {
        const float* Ab = Am + (I * 16) * LDA + K * 16;  // A_IK, [m][k]
        const float* Tb = Am + (K * 16) * LDA + J * 16;  // T_KJ, [k][n]
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4)
          x = Mfma<float>::mma(frag_k(Ab, LDA, k0, 16), frag_m(Tb, LDA, k0, 16), x);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Xs[J][(4 * (l >> 4) + i) * 16 + (l & 15)] = x[i];
    }
    __syncthreads();
    if (J < I) {
      f32x4 y = zero4();
      const float* Tii = Am + (I * 16) * LDA + I * 16;
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4)
        y = Mfma<float>::mma(frag_k(Tii, LDA, k0, 16), frag_m(&Xs[J][0], 16, k0, 16), y);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Am[(I * 16 + 4 * (l >> 4) + i) * LDA + J * 16 + (l & 15)] = -y[i];
    }
    __syncthreads();
  }

  // 5. Write the chunk record: Tm, Pm (operand type), gam (f32).
  char* rec = ws + ((size_t)bh * NC + chunk) * rec_bytes;
  OpT* Tg = reinterpret_cast<OpT*>(rec);
  OpT* Pg = Tg + C * C;
  float* Gg = reinterpret_cast<float*>(Pg + C * C);
  constexpr int VPRC = C / VN;
  for (int i = tid; i < C * VPRC; i += 256) {
    const int r = i / VPRC, cv = i % VPRC;
    ovec tv;
#pragma unroll
    for (int e = 0; e < VN; ++e) tv[e] = from_f32<OpT>(Am[r * LDA + cv * VN + e]);
    *reinterpret_cast<ovec*>(Tg + r * C + cv * VN) = tv;
    *reinterpret_cast<ovec*>(Pg + r * C + cv * VN) =
        *reinterpret_cast<const ovec*>(Ps + r * LDP + cv * VN);
  }
  if (tid < C) Gg[tid] = gam[tid];
}

// ---------------------------------------------------------------------------
// Kernel 2: sequential walk over the chunks of one (b, h), value slice of
// DVS columns.  S (Dk x DVS, f32) lives in MFMA accumulators; an operand-type
// copy of S^T sits in LDS as the B operand of K S0 and Q S0.
//
// Software pipeline: every global load of chunk c+1 (its K tile, the Q, Tm
// and Pm operand fragments, V, the log gates and beta) is issued into
// registers at the top of chunk c and only consumed one iteration later, so
// HBM/L2 latency overlaps the chunk's three dependent MFMA phases.  The K tile
// is double-buffered in LDS; three work-group barriers per chunk remain.
//
// Wave w owns one 16-token row tile (rt) of the chunk and OPW value tiles of
// it, and SPW 16x16 tiles of S.
// ---------------------------------------------------------------------------
template <class TIn, class TOut, int C, int DK, int DVS>
__global__ __launch_bounds__(256) void chunk_recur_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ beta,
    const float* state_in, float* state_out, TOut* __restrict__ out, int T,
    int H, int DV, int NC, int NS, float scale, const char* __restrict__ ws,
    size_t rec_bytes) {
  typedef typename OperandOf<TIn>::type OpT;
  typedef Mfma<OpT> M;
  typedef typename M::frag frag;
  typedef typename Vec16<TIn>::type vec;
  typedef typename Vec16<OpT>::type ovec;
  static_assert(sizeof(OpT) == sizeof(TIn), "operand and input sizes differ");
  constexpr int VN = Vec16<TIn>::N;
  constexpr int PAD = VN;
  constexpr int LDK = DK + PAD;
  constexpr int LDC = C + PAD;
  constexpr int RT = C / 16;        // token row tiles
  constexpr int NT = DVS / 16;      // value column tiles
  constexpr int MT = DK / 16;       // key row tiles of S
  constexpr int OT = RT * NT;       // token tiles (X, Y, U, O)
  constexpr int ST = MT * NT;       // state tiles
  constexpr int OPW = (OT + 3) / 4;
  constexpr int SPW = (ST + 3) / 4;
  constexpr int KQ = (DK + M::KSTEP - 1) / M::KSTEP;  // fragments over Dk
  constexpr int KC = (C + M::KSTEP - 1) / M::KSTEP;   // fragments over C
  constexpr int KV = (C * DK / VN + 255) / 256;       // K-tile vectors per thread

  __shared__ __align__(16) OpT Ks[2][C * LDK];  // K tile, double-buffered
  __shared__ __align__(16) OpT St[DVS * LDK];   // S^T (value-major)
  __shared__ __align__(16) OpT Yt[DVS * LDC];   // Y^T
  __shared__ __align__(16) OpT Ut[DVS * LDC];   // U^T
  __shared__ __align__(16) OpT Upt[DVS * LDC];  // (diag(exp(gam_C - gam)) U)^T
  __shared__ float gam[2][C], gexp[2][C], dec[2][C], bet[2][C];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = lane_id();
  int bh, slice;
  xcd_group_map(blockIdx.x, gridDim.x / NS, NS, &bh, &slice);
  const int b = bh / H, h = bh % H;
  const int col0 = slice * DVS;  // first value column of this slice
  const int rt = (wave * OPW) / NT;  // this wave's token row tile
  const bool has_rows = wave * OPW < OT;
  const size_t tok_stride = (size_t)H * DK;  // q/k elements between tokens
  const size_t vtok_stride = (size_t)H * DV;

  // ---- prefetch buffers (registers): raw loaded bits, converted at use ---
  // (a conversion right after a load would make the load complete at once)
  typedef typename RawFrag<TIn, M::KPL>::type qraw_t;
  vec kreg[KV];
  qraw_t qraw[KQ];
  frag tf[KC], pf[KC];
  uint32_t vreg[OPW][4];
  float greg = 0.f, breg = 0.f;

  auto prefetch = [&](int c) {
    const int t0 = c * C;
    const char* rec = ws + ((size_t)bh * NC + c) * rec_bytes;
    const OpT* Tg = reinterpret_cast<const OpT*>(rec);
    const OpT* Pg = Tg + C * C;
    const float* Gg = reinterpret_cast<const float*>(Pg + C * C);
    constexpr int VPR = DK / VN;
#pragma unroll
    for (int u = 0; u < KV; ++u) {
      const int i = tid + u * 256;
      const int r = i / VPR, cv = i % VPR;
      const int t = t0 + r;
      if (i < C * VPR && t < T) {
        kreg[u] = *reinterpret_cast<const vec*>(k + ((size_t)b * T + t) * tok_stride +
                                                (size_t)h * DK + cv * VN);
      } else {
#pragma unroll
        for (int e = 0; e < VN; ++e) kreg[u][e] = from_f32<TIn>(0.f);
      }
    }
    if (has_rows) {
      // Q operand fragments straight from global memory (rows of this tile).
      const int r = rt * 16 + (l & 15);
      const int t = t0 + r;
#pragma unroll
      for (int j = 0; j < KQ; ++j) {
        const int kk = j * M::KSTEP + (l >> 4) * M::KPL;
        if (t < T && kk < DK)
          qraw[j] = *reinterpret_cast<const qraw_t*>(
              q + ((size_t)b * T + t) * tok_stride + (size_t)h * DK + kk);
        else
          qraw[j] = RawFrag<TIn, M::KPL>::zero();
      }
      const int klim = (rt + 1) * 16;  // Tm, Pm are lower triangular
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        tf[j] = frag_k(Tg + rt * 16 * C, C, j * M::KSTEP, klim);
        pf[j] = frag_k(Pg + rt * 16 * C, C, j * M::KSTEP, klim);
      }
#pragma unroll
      for (int jj = 0; jj < OPW; ++jj) {
        const int x = wave * OPW + jj;
        const int cc = (x % NT) * 16 + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + rt * 16 + 4 * (l >> 4) + i;
          vreg[jj][i] = (x < OT && t < T)
                            ? load_raw32(v + ((size_t)b * T + t) * vtok_stride +
                                         (size_t)h * DV + col0 + cc)
                            : 0u;
        }
      }
    }
    if (tid < C) {
      const int t = t0 + tid;
      greg = Gg[tid];
      breg = (t < T) ? beta[((size_t)b * T + t) * H + h] : 0.f;
    }
  };

  // Initial state slice -> accumulators and the LDS operand copy.
  f32x4 S[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    S[j] = zero4();
    const int x = wave * SPW + j;
    if (x < ST) {
      const int mt = x / NT, nt = x % NT;
      const int cc = nt * 16 + (l & 15);
      if (state_in) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mt * 16 + 4 * (l >> 4) + i;
          S[j][i] = state_in[((size_t)bh * DK + r) * DV + col0 + cc];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        St[cc * LDK + mt * 16 + 4 * (l >> 4) + i] = from_f32<OpT>(S[j][i]);
    }
  }

  // Output tiles of the previous chunk, stored at the top of the next chunk
  // ahead of its prefetch: vmcnt counts stores too, so a store issued late in
  // a chunk would otherwise make the next loop-top wait cover its latency.
  f32x4 Opend[OPW];
  int t0_pend = -1;
  auto store_pending = [&]() {
    if (t0_pend < 0 || !has_rows) return;
#pragma unroll
    for (int jj = 0; jj < OPW; ++jj) {
      const int x = wave * OPW + jj;
      if (x < OT) {
        const int cc = (x % NT) * 16 + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0_pend + rt * 16 + 4 * (l >> 4) + i;
          if (t < T)
            out[((size_t)b * T + t) * vtok_stride + (size_t)h * DV + col0 + cc] =
                from_f32<TOut>(Opend[jj][i]);
        }
      }
    }
  };

  if (NC > 0) prefetch(0);

  for (int c = 0; c < NC; ++c) {
    const int t0 = c * C;
    const int buf = c & 1;
    OpT* Kb = Ks[buf];
    // Commit chunk c's K tile and gates to LDS.
    {
      constexpr int VPR = DK / VN;
#pragma unroll
      for (int u = 0; u < KV; ++u) {
        const int i = tid + u * 256;
        if (i < C * VPR) {
          const int r = i / VPR, cv = i % VPR;
          ovec o;
#pragma unroll
          for (int e = 0; e < VN; ++e) o[e] = from_f32<OpT>(to_f32(kreg[u][e]));
          *reinterpret_cast<ovec*>(Kb + r * LDK + cv * VN) = o;
        }
      }
    }
    if (tid < C) {
      gam[buf][tid] = greg;
      gexp[buf][tid] = __expf(greg);
      bet[buf][tid] = breg;
    }
    // Chunk c's register operands; then issue chunk c+1's loads.
    frag cq[KQ], ct[KC], cp[KC];
    float cv4[OPW][4];
#pragma unroll
    for (int j = 0; j < KQ; ++j) cq[j] = RawFrag<TIn, M::KPL>::template to_frag<OpT>(qraw[j]);
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      ct[j] = tf[j];
      cp[j] = pf[j];
    }
#pragma unroll
    for (int jj = 0; jj < OPW; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) cv4[jj][i] = raw32_to_f32<TIn>(vreg[jj][i]);
    const float my_gam = greg;
    store_pending();
    if (c + 1 < NC) prefetch(c + 1);
    __syncthreads();  // (1) K tile, gates, and S^T of the previous chunk visible
    if (tid < C) dec[buf][tid] = __expf(gam[buf][C - 1] - my_gam);

    // Phase A: X = K S0, QS = Q S0; Y = diag(beta) (V - diag(g) X) -> Y^T.
    f32x4 QS[OPW];
#pragma unroll
    for (int jj = 0; jj < OPW; ++jj) {
      QS[jj] = zero4();
      const int x = wave * OPW + jj;
      if (x < OT) {
        const int nt = x % NT;
        f32x4 X = zero4();
        const OpT* Kr = Kb + rt * 16 * LDK;
        const OpT* Sr = St + nt * 16 * LDK;
#pragma unroll
        for (int j = 0; j < KQ; ++j) {
          const frag sb = frag_k(Sr, LDK, j * M::KSTEP, DK);
          X = M::mma(frag_k(Kr, LDK, j * M::KSTEP, DK), sb, X);
          QS[jj] = M::mma(cq[j], sb, QS[jj]);
        }
        const int cc = nt * 16 + (l & 15);
        OpT yv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rt * 16 + 4 * (l >> 4) + i;
          yv[i] = from_f32<OpT>(bet[buf][r] * (cv4[jj][i] - gexp[buf][r] * X[i]));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Yt[cc * LDC + rt * 16 + 4 * (l >> 4) + i] = yv[i];
      }
    }
    __syncthreads();  // (2) Y^T and dec visible

    // Phase B: U = Tm Y (Tm lower triangular: only k < 16 (rt + 1)).
    const int klim = (rt + 1) * 16;
#pragma unroll
    for (int jj = 0; jj < OPW; ++jj) {
      const int x = wave * OPW + jj;
      if (x < OT) {
        const int nt = x % NT;
        f32x4 U = zero4();
        const OpT* Yr = Yt + nt * 16 * LDC;
#pragma unroll
        for (int j = 0; j < KC; ++j)
          if (j * M::KSTEP < klim) U = M::mma(ct[j], frag_k(Yr, LDC, j * M::KSTEP, klim), U);
        const int cc = nt * 16 + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rt * 16 + 4 * (l >> 4) + i;
          Ut[cc * LDC + r] = from_f32<OpT>(U[i]);
          Upt[cc * LDC + r] = from_f32<OpT>(dec[buf][r] * U[i]);
        }
      }
    }
    __syncthreads();  // (3) U^T visible

    // Phase C1: O = diag(scale g) QS + Pm U.
#pragma unroll
    for (int jj = 0; jj < OPW; ++jj) {
      const int x = wave * OPW + jj;
      if (x < OT) {
        const int nt = x % NT;
        f32x4 O;
#pragma unroll
        for (int i = 0; i < 4; ++i) O[i] = scale * gexp[buf][rt * 16 + 4 * (l >> 4) + i] * QS[jj][i];
        const OpT* Ur = Ut + nt * 16 * LDC;
#pragma unroll
        for (int j = 0; j < KC; ++j)
          if (j * M::KSTEP < klim) O = M::mma(cp[j], frag_k(Ur, LDC, j * M::KSTEP, klim), O);
        Opend[jj] = O;
      }
    }
    t0_pend = t0;
    // Phase C2: S = g_C S + K^T diag(exp(gam_C - gam)) U.
    const float gc = gexp[buf][C - 1];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int x = wave * SPW + j;
      if (x < ST) {
        const int mt = x / NT, nt = x % NT;
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = gc * S[j][i];
        const OpT* Kc = Kb + mt * 16;  // K^T rows = columns of the K tile
        const OpT* Ur = Upt + nt * 16 * LDC;
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
          acc = M::mma(frag_m(Kc, LDK, kk * M::KSTEP, C), frag_k(Ur, LDC, kk * M::KSTEP, C), acc);
        S[j] = acc;
        const int cc = nt * 16 + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          St[cc * LDK + mt * 16 + 4 * (l >> 4) + i] = from_f32<OpT>(acc[i]);
      }
    }
    // No barrier here: the next chunk writes the other K buffer and gate
    // slot, and its first barrier orders this chunk's S^T writes before use.
  }
  store_pending();

  // Final state slice.
  if (state_out) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int x = wave * SPW + j;
      if (x < ST) {
        const int mt = x / NT, nt = x % NT;
        const int cc = nt * 16 + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mt * 16 + 4 * (l >> 4) + i;
          state_out[((size_t)bh * DK + r) * DV + col0 + cc] = S[j][i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launch: kernel 1 over all chunks, then kernel 2 over (b, h, value slice).
// ---------------------------------------------------------------------------
static int pick_slices(int BH, int DV) {
  // Smallest power-of-two split that fills the chip (>= 256 work-groups),
  // keeping slices at least 16 columns and at most 64.
  int ns = 1;
  while (DV / ns > 64) ns *= 2;
  while ((long)BH * ns < 256 && DV / ns > 16) ns *= 2;
  return ns;
}

template <class TIn, class TOut, int C, int DK, int DVS>
static hipError_t launch_recur(const PrefillArgs& p, int NC, int NS, size_t rb) {
  const int grid = p.B * p.H * NS;
  hipLaunchKernelGGL((chunk_recur_kernel<TIn, TOut, C, DK, DVS>), dim3(grid), dim3(256), 0,
                     (hipStream_t)p.stream, (const TIn*)p.q, (const TIn*)p.k,
                     (const TIn*)p.v, p.beta, p.state_in, p.state_out, (TOut*)p.out,
                     p.T, p.H, p.Dv, NC, NS, p.scale, (const char*)p.workspace, rb);
  return hipGetLastError();
}

template <class TIn, class TOut, int C, int DK>
static hipError_t launch_recur_dvs(const PrefillArgs& p, int NC, int NS, size_t rb) {
  switch (p.Dv / NS) {
    case 16: return launch_recur<TIn, TOut, C, DK, 16>(p, NC, NS, rb);
    case 32: return launch_recur<TIn, TOut, C, DK, 32>(p, NC, NS, rb);
    case 64: return launch_recur<TIn, TOut, C, DK, 64>(p, NC, NS, rb);
  }
  return hipErrorInvalidValue;
}

template <class TIn, int C, int DK>
static hipError_t launch_prefill_t(const PrefillArgs& p) {
  const int NC = (p.T + C - 1) / C;
  const size_t rb = prefill_record_bytes(C, sizeof(TIn) == 2);
  if (NC > 0) {
    hipLaunchKernelGGL((chunk_prep_kernel<TIn, C, DK>), dim3(p.B * p.H * NC), dim3(256), 0,
                       (hipStream_t)p.stream, (const TIn*)p.q, (const TIn*)p.k, p.alpha,
                       p.beta, p.T, p.H, NC, p.scale, (char*)p.workspace, rb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int NS = pick_slices(p.B * p.H, p.Dv);
  if constexpr (sizeof(TIn) == 4) {
    return launch_recur_dvs<TIn, float, C, DK>(p, NC, NS, rb);
  } else {
    return p.out_bf16 ? launch_recur_dvs<TIn, bf16, C, DK>(p, NC, NS, rb)
                      : launch_recur_dvs<TIn, float, C, DK>(p, NC, NS, rb);
  }
}

template <class TIn, int C>
static hipError_t launch_prefill_dk(const PrefillArgs& p) {
  switch (p.Dk) {
    case 16: return launch_prefill_t<TIn, C, 16>(p);
    case 32: return launch_prefill_t<TIn, C, 32>(p);
    case 64: return launch_prefill_t<TIn, C, 64>(p);
    case 128: return launch_prefill_t<TIn, C, 128>(p);
  }
  return hipErrorInvalidValue;
}

template <class TIn>
static hipError_t launch_prefill_c(const PrefillArgs& p) {
  switch (p.chunk) {
    case 16: return launch_prefill_dk<TIn, 16>(p);
    case 32: return launch_prefill_dk<TIn, 32>(p);
    case 64: return launch_prefill_dk<TIn, 64>(p);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& p) {
  if (p.B * p.H == 0) return hipSuccess;
  if (p.taps_q) {
    // The fused convolution exists in the per-head kernels only.
    if (p.T > 0 && !prefill_head_conv_supported(p)) return hipErrorInvalidValue;
    if (p.T > 0) return launch_prefill_head(p);
  }
  if (prefill_head_supported(p)) return launch_prefill_head(p);
  // The other kernels address dense [B, T, ...] tensors.
  if (p.T > 0 && p.B > 1 && p.seq_stride > 0 && p.seq_stride != p.T) return hipErrorInvalidValue;
  return p.bf16 ? launch_prefill_c<bf16>(p) : launch_prefill_c<float>(p);
}

}  // namespace gdn
