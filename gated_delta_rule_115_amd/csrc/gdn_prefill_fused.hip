// Single-pass chunked GDN prefill for gfx950: bf16 inputs, d_k = 128,
// chunks of 64 tokens, value dimension split into 16-column slices.
//
// Method: "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 3.1.2 (S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1}
// + beta_t k_t v_t^T, o_t = scale * S_t^T q_t), computed chunk by chunk with the
// exact WY/UT rewrite.  For a chunk entering with state S (gam_r = cumulative
// log gate, g_r = exp(gam_r)):
//   A_ri = beta_r exp(gam_r - gam_i) k_r.k_i   (i < r),   Tm = (I + A)^-1
//   Pm_ri = scale exp(gam_r - gam_i) q_r.k_i    (i <= r)
//   Y = diag(beta) (V - diag(g) K S),   U = Tm Y
//   O = diag(scale g) Q S + Pm U
//   S <- g_C S + K^T diag(exp(gam_C - gam)) U
//
// One work-group of 8 waves owns one (batch, head, 16-column value slice) and
// walks all chunks of the sequence.  q, k, v, alpha, beta are read from HBM
// once and o is written once: nothing goes through a workspace.  The slices
// of one head sit on one XCD and share its L2 copy of the q/k tiles.
//
// Wave roles (wave-uniform branches; every wave passes the same barriers):
//   state waves 0..3  carry S in MFMA accumulators, split by key rows: wave w
//                     owns rows 32w .. 32w+31.  Per chunk: partial K S and
//                     Q S over its rows -> (LDS) -> token tile w reduces them,
//                     forms Y -> (LDS) -> U = Tm Y for tile w -> (LDS) -> output
//                     tile w and the S update of its rows.
//   prep waves 4..7   run one chunk ahead: global loads of chunk c+2 into
//                     registers, commit of chunk c+1's tiles and gates to LDS,
//                     the Gram products of chunk c+1 (each wave a fixed set of
//                     five 16x16 tiles), A and Pm, and the blocked triangular
//                     inverse Tm: each diagonal 16x16 block as
//                     (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8) (L is
//                     strictly lower, so L^16 = 0) with 16x16x16 MFMAs, then
//                     two levels of block products for the off-diagonal blocks.
// Each chunk is four phases separated by work-group barriers:
//   P1  state: partial K S, Q S (chunk c)      prep: commit c+1, load c+2, inverse level 1 (c)
//   P2  state: reduce, Y                       prep: inverse level 2 (c), Gram c+1 (k 0..63)
//   P3  state: U = Tm Y                        prep: Gram c+1 (k 64..127)
//   P4  state: O, S update                     prep: A, Pm, diagonal Tm blocks of c+1
//
// Operand layouts.  A 16x16 MFMA result tile is held by lane l as rows
// 4 (l/16) .. +3 of column l % 16 (the accumulator layout); a matrix M in
// accumulator layout is M^T in A-operand layout.  The C x C matrices (A, Pm,
// Tm) are kept in LDS as [block row][block col][lane][4] in the layout their
// consumer feeds to the MFMA, so every access is one 8-byte lane-contiguous
// LDS operation.  The Gram tiles come out in that layout directly: K K^T is
// symmetric, and Q K^T is computed as (K Q^T)^T.  The inverse carries every
// block in both orientations (M N = mfma(M^T, N), (M N)^T = mfma(N, M^T) on
// accumulator-layout fragments), so no transpose passes through LDS.
//
// v_mfma_f32_16x16x32_f16 sums over 32 contraction values, 8 per lane; which
// logical index a lane's j-th value stands for is free as long as A and B
// agree.  On the state path lane group q = lane / 16 carries the indices
// {4q .. 4q+3} and {16 + 4q .. 16 + 4q + 3} of each 32-wide step, which is how
// two stacked accumulator tiles hold their rows: S, Y, U and the decayed U
// feed the next product straight from registers.  The K and Q tiles store
// their key columns permuted to match (within each group of 32, logical
// 16h + 4q + i sits at 8q + 4h + i), so those operands are single 16-byte
// reads; the Gram products contract over the permuted columns unchanged.
//
// Gate ratios exp(gam_r - gam_c) are formed as exp(gam_r) * exp(-gam_c) from
// per-token tables when the chunk's log-gate range is within 80 (no overflow
// possible); otherwise the chunk falls back to one exp per element.
//
// Precision: bf16 inputs are converted to f16 exactly (unit-scale values);
// every product takes f16 operands with f32 accumulation; S is f32.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int FC = 64;          // tokens per chunk
constexpr int FDK = 128;        // key dimension
constexpr int FLD = FDK + 8;    // f16 row stride of the K / Q tiles (272 B)
constexpr int NTHR = 512;
constexpr float kWideGate = -80.f;  // log-gate range beyond which exps are exact

typedef _Float16 h16;
typedef h16 h16x4 __attribute__((ext_vector_type(4)));
typedef h16 h16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

struct __align__(16) FusedSmem {
  h16 K[2][FC * FLD];      // K tiles of chunks c and c+1 (f16, [token][permuted key])
  h16 Q[2][FC * FLD];      // Q tiles
  f32x4 XP[4][4][64];      // partial K S: [state wave][token tile][lane]
  f32x4 QP[4][4][64];      // partial Q S
  f32x4 V[2][4][64];       // value slice, accumulator layout: [tile][lane][row]
  h16x4 Y[4][64];          // Y tiles, accumulator layout
  h16x4 U[4][64];          // U tiles
  h16x4 Ud[4][64];         // diag(exp(gam_C - gam)) U tiles
  h16x4 Af[4][4][64];      // A blocks (I, J), J < I, A-operand layout
  h16x4 Tf[4][4][64];      // Tm blocks, A-operand layout; upper blocks stay 0
  h16x4 TBf[4][4][64];     // Tm blocks, accumulator layout (inverse's right factors)
  h16x4 Pmf[4][4][64];     // Pm blocks, A-operand layout; upper blocks stay 0
  float gam[2][FC], gpos[2][FC], gneg[2][FC], bet[2][FC], dec[2][FC];
  int wide[2];             // the chunk's log-gate range exceeds kWideGate
};

__device__ __forceinline__ f32x4 mfma32(h16x8 a, h16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(h16x4 a, h16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ h16x8 cat8(h16x4 lo, h16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ h16x4 cvt4(f32x4 x) {
  h16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (h16)x[i];
  return r;
}
__device__ __forceinline__ f32x4 ldf4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
// Physical column of logical key column c in the K / Q tiles.
__device__ __forceinline__ int perm_col(int c) {
  return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}

// (I + L)^-1 and its transpose for a nilpotent 16x16 L (L^16 = 0), from L and
// L^T in accumulator layout (f32).  Every product is carried in both
// orientations: with M, M^T in accumulator layout, M N = mfma(M^T, N) and
// (M N)^T = mfma(N, M^T).
__device__ __forceinline__ void inv_unit16(f32x4 Lf, f32x4 LTf, int lr, int lq, f32x4& T,
                                           f32x4& TT) {
  const h16x4 lo = cvt4(Lf), lt = cvt4(LTf);
  const f32x4 L2 = mfma16(lt, lo, zero4());
  const f32x4 L2T = mfma16(lo, lt, zero4());
  const h16x4 l2 = cvt4(L2), l2t = cvt4(L2T);
  const f32x4 L4 = mfma16(l2t, l2, zero4());
  const f32x4 L4T = mfma16(l2, l2t, zero4());
  const f32x4 LL2 = mfma16(lt, l2, zero4());   // L L^2
  const f32x4 LL2T = mfma16(l2, lt, zero4());  // (L L^2)^T
  const h16x4 l4 = cvt4(L4), l4t = cvt4(L4T);
  const h16x4 l8 = cvt4(mfma16(l4t, l4, zero4()));
  f32x4 P1, P1T;  // (I - L)(I + L^2) = I - L + L^2 - L^3 and its transpose
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float id = (4 * lq + i == lr) ? 1.f : 0.f;
    P1[i] = id - Lf[i] + L2[i] - LL2[i];
    P1T[i] = id - LTf[i] + L2T[i] - LL2T[i];
  }
  const h16x4 p1t = cvt4(P1T);
  const f32x4 P2 = P1 + mfma16(p1t, l4, zero4());    // P1 (I + L^4)
  const f32x4 P2T = P1T + mfma16(l4, p1t, zero4());
  const h16x4 p2t = cvt4(P2T);
  T = P2 + mfma16(p2t, l8, zero4());                 // P2 (I + L^8)
  TT = P2T + mfma16(l8, p2t, zero4());
}

struct PrepArgs {
  const bf16* qh;
  const bf16* kh;
  const bf16* vh;
  const float* ah;
  const float* bth;
  size_t qk_tok, v_tok;
  int T, H, NC;
  float scale;
};

// Prep wave W (0..3).  Gram tiles: K K^T (W = 0, 1) or Q K^T (W = 2, 3), row
// blocks {3, 0} (W even: tiles (3,0..3) and (0,0)) or {2, 1} (W odd: tiles
// (2,0..2) and (1,0..1)).  W = 0 also loads and scans the gates; W = 0 and 1
// finish the triangular inverse.
template <int W>
__device__ __forceinline__ void prep_loop(FusedSmem& sm, const PrepArgs& a, int l) {
  constexpr bool GQ = W >= 2;
  constexpr int RA = (W & 1) ? 2 : 3;
  constexpr int RB = (W & 1) ? 1 : 0;
  const int lr = l & 15, lq = l >> 4;
  const int pt = W * 64 + l;  // prep thread 0..255
  const int T = a.T, NC = a.NC;

  // Per-thread element offsets of its share of a chunk (token row in the
  // chunk times the token stride, plus the column): 4 q/k vectors, 1 v quad.
  int off_qk[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int vi = pt + 256 * u;
    off_qk[u] = (vi >> 4) * (int)a.qk_tok + (vi & 15) * 8;
  }
  const int off_v = (pt >> 2) * (int)a.v_tok + (pt & 3) * 4;

  bf16x8 kreg[4], qreg[4];
  bf16x4_t vreg;
  float areg = 1.f, breg = 0.f;

  auto prefetch = [&](int c) {
    const int t0 = c * FC;
    const bf16* kc = a.kh + (size_t)t0 * a.qk_tok;
    const bf16* qc = a.qh + (size_t)t0 * a.qk_tok;
    const bf16* vc = a.vh + (size_t)t0 * a.v_tok;
    if (t0 + FC <= T) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kreg[u] = *reinterpret_cast<const bf16x8*>(kc + off_qk[u]);
        qreg[u] = *reinterpret_cast<const bf16x8*>(qc + off_qk[u]);
      }
      vreg = *reinterpret_cast<const bf16x4_t*>(vc + off_v);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (t0 + ((pt + 256 * u) >> 4) < T) {
          kreg[u] = *reinterpret_cast<const bf16x8*>(kc + off_qk[u]);
          qreg[u] = *reinterpret_cast<const bf16x8*>(qc + off_qk[u]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kreg[u][e] = (bf16)0.f;
            qreg[u][e] = (bf16)0.f;
          }
        }
      }
      if (t0 + (pt >> 2) < T) {
        vreg = *reinterpret_cast<const bf16x4_t*>(vc + off_v);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) vreg[e] = (bf16)0.f;
      }
    }
    if (W == 0) {
      const int t = t0 + l;
      areg = (t < T) ? a.ah[(size_t)t * a.H] : 1.f;
      breg = (t < T) ? a.bth[(size_t)t * a.H] : 0.f;
    }
  };

  // Registers -> LDS for a chunk: K, Q tiles as f16 (key columns permuted),
  // the value slice in accumulator layout, and (W = 0) the gate tables.
  auto commit = [&](int nb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int vi = pt + 256 * u;
      const int row = vi >> 4, c0 = (vi & 15) * 8;
      const int p0 = row * FLD + perm_col(c0), p1 = row * FLD + perm_col(c0 + 4);
      h16x4 k0, k1, q0, q1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k0[e] = (h16)(float)kreg[u][e];
        k1[e] = (h16)(float)kreg[u][4 + e];
        q0[e] = (h16)(float)qreg[u][e];
        q1[e] = (h16)(float)qreg[u][4 + e];
      }
      *reinterpret_cast<h16x4*>(sm.K[nb] + p0) = k0;
      *reinterpret_cast<h16x4*>(sm.K[nb] + p1) = k1;
      *reinterpret_cast<h16x4*>(sm.Q[nb] + p0) = q0;
      *reinterpret_cast<h16x4*>(sm.Q[nb] + p1) = q1;
    }
    {
      const int row = pt >> 2, c4 = (pt & 3) * 4;
      const int rt = row >> 4, qq = (row & 15) >> 2, ii = row & 3;
      float* vb = reinterpret_cast<float*>(&sm.V[nb][rt][0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) vb[(16 * qq + c4 + e) * 4 + ii] = (float)vreg[e];
    }
    if (W == 0) {
      float la = logf(areg);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(la, off);
        if (l >= off) la += y;
      }
      const float gl = __shfl(la, 63);
      const bool wide = gl < kWideGate;
      sm.gam[nb][l] = la;
      sm.gpos[nb][l] = __expf(la);
      sm.gneg[nb][l] = wide ? 0.f : __expf(-la);
      sm.bet[nb][l] = breg;
      sm.dec[nb][l] = __expf(gl - la);
      if (l == 0) sm.wide[nb] = wide ? 1 : 0;
    }
  };

  // Gram accumulators.  Tile (R, C) is computed as mfma(K_C, X_R) with X = K
  // (W = 0, 1) or Q (W = 2, 3): the result is (X K^T) restricted to the tile,
  // in A-operand layout (lane holds element (16R + lr, 16C + 4 lq + i)); for
  // K K^T this uses its symmetry.
  f32x4 GA[RA + 1], GB[RB + 1];

  auto gram_steps = [&](int nb, int k_begin, int k_end) {
    const h16* Kb = sm.K[nb];
    const h16* Qb = sm.Q[nb];
    for (int ks = k_begin; ks < k_end; ++ks) {
      const int kc = ks * 32 + lq * 8;
      h16x8 kf[RA + 1];
#pragma unroll
      for (int c = 0; c <= RA; ++c)
        kf[c] = *reinterpret_cast<const h16x8*>(Kb + (16 * c + lr) * FLD + kc);
      const h16x8 fa = GQ ? *reinterpret_cast<const h16x8*>(Qb + (16 * RA + lr) * FLD + kc)
                          : kf[RA];
      const h16x8 fb = GQ ? *reinterpret_cast<const h16x8*>(Qb + (16 * RB + lr) * FLD + kc)
                          : kf[RB];
#pragma unroll
      for (int c = 0; c <= RA; ++c) GA[c] = mfma32(kf[c], fa, GA[c]);
#pragma unroll
      for (int c = 0; c <= RB; ++c) GB[c] = mfma32(kf[c], fb, GB[c]);
    }
  };

  // Tile (R, C) -> Pm (W = 2, 3), an off-diagonal block of A (C < R), or the
  // diagonal block of A, whose inverse is written to Tm in both layouts.
  auto finish_tile = [&](int nb, bool wide, int R, int C, f32x4 G) {
    const float* gm = sm.gam[nb];
    const float* bt = sm.bet[nb];
    const int r = 16 * R + lr;         // this lane's row
    const int cb = 16 * C + 4 * lq;    // first of this lane's 4 columns
    const float rowf = GQ ? a.scale : bt[r];
    if (GQ || C < R) {
      f32x4 f;
      if (!wide) {
        const float rs = rowf * sm.gpos[nb][r];
        const f32x4 gn = ldf4(&sm.gneg[nb][cb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = rs * gn[i];
      } else {
        const float gr = gm[r];
        const f32x4 gc = ldf4(&gm[cb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = rowf * __expf(gr - gc[i]);
      }
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (C < R || cb + i <= r) ? f[i] * G[i] : 0.f;
      if (GQ) {
        sm.Pmf[R][C][l] = cvt4(x);
      } else {
        sm.Af[R][C][l] = cvt4(x);
      }
    } else {
      // Diagonal block: G is symmetric, so lane (lq, lr) holds G at both
      // (4 lq + i, lr) and (lr, 4 lq + i).  L in accumulator layout takes
      // element (4 lq + i, lr); L^T takes element (lr, 4 lq + i) of L.
      const int rb = 16 * R;
      const f32x4 bv = ldf4(&bt[rb + 4 * lq]);
      f32x4 fL, fT;
      if (!wide) {
        const f32x4 gpv = ldf4(&sm.gpos[nb][rb + 4 * lq]);
        const f32x4 gnv = ldf4(&sm.gneg[nb][rb + 4 * lq]);
        const float gpl = sm.gpos[nb][rb + lr], gnl = sm.gneg[nb][rb + lr];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fL[i] = bv[i] * gpv[i] * gnl;
          fT[i] = rowf * gpl * gnv[i];
        }
      } else {
        const f32x4 gv = ldf4(&gm[rb + 4 * lq]);
        const float gll = gm[rb + lr];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fL[i] = bv[i] * __expf(gv[i] - gll);
          fT[i] = rowf * __expf(gll - gv[i]);
        }
      }
      f32x4 Lf, LTf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Lf[i] = (4 * lq + i > lr) ? fL[i] * G[i] : 0.f;
        LTf[i] = (lr > 4 * lq + i) ? fT[i] * G[i] : 0.f;
      }
      f32x4 Tb, TTb;
      inv_unit16(Lf, LTf, lr, lq, Tb, TTb);
      sm.Tf[R][R][l] = cvt4(TTb);
      sm.TBf[R][R][l] = cvt4(Tb);
    }
  };

  auto finish = [&](int nb) {
    const bool wide = __builtin_amdgcn_readfirstlane(sm.wide[nb]) != 0;
#pragma unroll
    for (int c = 0; c <= RA; ++c) finish_tile(nb, wide, RA, c, GA[c]);
#pragma unroll
    for (int c = 0; c <= RB; ++c) finish_tile(nb, wide, RB, c, GB[c]);
  };

  // Level 1: T_10 = -T_11 A_10 T_00 (W = 0), T_32 = -T_33 A_32 T_22 (W = 1).
  auto inverse_level1 = [&]() {
    constexpr int I = (W == 0) ? 1 : 3, J = I - 1;
    const h16x4 x = cvt4(mfma16(sm.Af[I][J][l], sm.TBf[J][J][l], zero4()));  // A_IJ T_JJ
    const h16x4 tii = sm.Tf[I][I][l];
    sm.TBf[I][J][l] = cvt4(-mfma16(tii, x, zero4()));  // -T_II X
    sm.Tf[I][J][l] = cvt4(-mfma16(x, tii, zero4()));   // -(X^T T_II^T)
  };

  // Level 2: lower-left 32x32 block -T22 (A21 T11), column block j = W, in
  // A-operand layout (the Tm consumers' layout).
  auto inverse_level2 = [&]() {
    constexpr int j = W;
    f32x4 Z2 = zero4(), Z3 = zero4();
#pragma unroll
    for (int K = j; K < 2; ++K) {
      const h16x4 tb = sm.TBf[K][j][l];
      Z2 = mfma16(sm.Af[2][K][l], tb, Z2);
      Z3 = mfma16(sm.Af[3][K][l], tb, Z3);
    }
    const h16x4 z2 = cvt4(Z2), z3 = cvt4(Z3);
    sm.Tf[2][j][l] = cvt4(-mfma16(z2, sm.Tf[2][2][l], zero4()));
    sm.Tf[3][j][l] =
        cvt4(-(mfma16(z2, sm.Tf[3][2][l], zero4()) + mfma16(z3, sm.Tf[3][3][l], zero4())));
  };

  prefetch(0);
  for (int c = 0; c <= NC; ++c) {
    // Iteration c prepares chunk c (tiles, gates, Gram, A, Pm, diagonal Tm
    // blocks) and finishes the inverse of chunk c - 1.
    const int nb = c & 1;
    const bool prev = c >= 1;
    const bool cur = c < NC;
    // P1: commit chunk c, load chunk c + 1, inverse level 1 of chunk c - 1.
    if (cur) commit(nb);
    if (c + 1 < NC) prefetch(c + 1);
    if (W < 2 && prev) inverse_level1();
    __syncthreads();
    // P2: inverse level 2 of chunk c - 1; first half of chunk c's Gram.
    if (W < 2 && prev) inverse_level2();
    if (cur) {
#pragma unroll
      for (int j = 0; j <= RA; ++j) GA[j] = zero4();
#pragma unroll
      for (int j = 0; j <= RB; ++j) GB[j] = zero4();
      gram_steps(nb, 0, 2);
    }
    __syncthreads();
    // P3: second half of the Gram.
    if (cur) gram_steps(nb, 2, 4);
    __syncthreads();
    // P4: A, Pm and the diagonal Tm blocks of chunk c.
    if (cur) finish(nb);
    __syncthreads();
  }
}

template <class TOut>
__global__ __launch_bounds__(NTHR) void prefill_fused_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k,
    const bf16* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* state_in, float* state_out,
    TOut* __restrict__ out, int T, int H, int DV, int NC, int NS, float scale) {
  __shared__ FusedSmem sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int lr = l & 15, lq = l >> 4;
  const int w4 = wave & 3;  // index within the role group

  int bh, slice;
  xcd_group_map(blockIdx.x, gridDim.x / NS, NS, &bh, &slice);
  const int b = bh / H, h = bh % H;
  const int col0 = slice * 16;
  const size_t qk_tok = (size_t)H * FDK;  // elements between consecutive tokens
  const size_t v_tok = (size_t)H * DV;

  // Upper blocks of Tf and Pmf are read as zeros by the lower-triangular
  // products and never written afterwards.
  {
    h16x4* tz = &sm.Tf[0][0][0];
    h16x4* pz = &sm.Pmf[0][0][0];
    for (int i = tid; i < 16 * 64; i += NTHR) {
      tz[i] = h16x4{0, 0, 0, 0};
      pz[i] = h16x4{0, 0, 0, 0};
    }
  }
  __syncthreads();

  if (wave >= 4) {
    PrepArgs pa;
    pa.qh = q + (size_t)b * T * qk_tok + (size_t)h * FDK;
    pa.kh = k + (size_t)b * T * qk_tok + (size_t)h * FDK;
    pa.vh = v + (size_t)b * T * v_tok + (size_t)h * DV + col0;
    pa.ah = alpha + (size_t)b * T * H + h;
    pa.bth = beta + (size_t)b * T * H + h;
    pa.qk_tok = qk_tok;
    pa.v_tok = v_tok;
    pa.T = T;
    pa.H = H;
    pa.NC = NC;
    pa.scale = scale;
    switch (w4) {
      case 0: prep_loop<0>(sm, pa, l); break;
      case 1: prep_loop<1>(sm, pa, l); break;
      case 2: prep_loop<2>(sm, pa, l); break;
      default: prep_loop<3>(sm, pa, l); break;
    }
    return;
  }

  // ===================== state waves =====================
  // S rows 32 w4 + 16 hh + 4 lq + i, column col0 + lr.
  TOut* oh = out + (size_t)b * T * v_tok + (size_t)h * DV + col0;
  f32x4 S[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 32 * w4 + 16 * hh + 4 * lq + i;
      S[hh][i] = state_in ? state_in[((size_t)bh * FDK + row) * DV + col0 + lr] : 0.f;
    }
  }
  // K^T gather columns: logical key rows 32 w4 + 16 hh + lr of the S update.
  int kcol[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) kcol[hh] = perm_col(32 * w4 + 16 * hh + lr);
  const int r0 = 16 * w4 + 4 * lq;  // this lane's 4 token rows: r0 .. r0 + 3

  f32x4 QSr = zero4();
  h16x8 pmf[2];
  h16x8 ktf[2][2];
  for (int c = 0; c <= NC; ++c) {
    // Iteration c works on chunk c - 1 (the prep waves run one chunk ahead,
    // so the first iteration only waits for them).
    const int cc = c - 1;
    const int cb = cc & 1;
    const bool run = cc >= 0;
    // P1: partial K S and Q S over this wave's 32 key rows.
    if (run) {
      const h16x8 sb = cat8(cvt4(S[0]), cvt4(S[1]));
      const h16* Kb = sm.K[cb];
      const h16* Qb = sm.Q[cb];
      const int kc = 32 * w4 + 8 * lq;  // permuted columns of this wave's keys
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int row = 16 * rt + lr;
        const h16x8 ka = *reinterpret_cast<const h16x8*>(Kb + row * FLD + kc);
        const h16x8 qa = *reinterpret_cast<const h16x8*>(Qb + row * FLD + kc);
        sm.XP[w4][rt][l] = mfma32(ka, sb, zero4());
        sm.QP[w4][rt][l] = mfma32(qa, sb, zero4());
      }
    }
    __syncthreads();
    // P2: reduce token tile w4; Y = diag(beta) (V - diag(g) K S).
    if (run) {
      f32x4 X = sm.XP[0][w4][l];
      QSr = sm.QP[0][w4][l];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        X += sm.XP[w][w4][l];
        QSr += sm.QP[w][w4][l];
      }
      const f32x4 Vv = sm.V[cb][w4][l];
      const f32x4 bv = ldf4(&sm.bet[cb][r0]);
      const f32x4 gv = ldf4(&sm.gpos[cb][r0]);
      h16x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = (h16)(bv[i] * (Vv[i] - gv[i] * X[i]));
      sm.Y[w4][l] = y;
      // K^T operands of this chunk's S update (key rows of this wave).
      const h16* Kb = sm.K[cb];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ktf[hh][jp][i] = Kb[(32 * jp + 4 * lq + i) * FLD + kcol[hh]];
            ktf[hh][jp][4 + i] = Kb[(32 * jp + 16 + 4 * lq + i) * FLD + kcol[hh]];
          }
        }
      }
    }
    __syncthreads();
    // P3: U = Tm Y for token tile w4 (Tm lower triangular).
    if (run) {
      f32x4 U = zero4();
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        pmf[jp] = cat8(sm.Pmf[w4][2 * jp][l], sm.Pmf[w4][2 * jp + 1][l]);
        if (jp == 0 || w4 >= 2) {
          const h16x8 ta = cat8(sm.Tf[w4][2 * jp][l], sm.Tf[w4][2 * jp + 1][l]);
          U = mfma32(ta, cat8(sm.Y[2 * jp][l], sm.Y[2 * jp + 1][l]), U);
        }
      }
      const f32x4 dv = ldf4(&sm.dec[cb][r0]);
      h16x4 u16, ud16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u16[i] = (h16)U[i];
        ud16[i] = (h16)(dv[i] * U[i]);
      }
      sm.U[w4][l] = u16;
      sm.Ud[w4][l] = ud16;
    }
    __syncthreads();
    // P4: O = diag(scale g) Q S + Pm U;  S <- g_C S + K^T diag(dec) U.
    if (run) {
      const f32x4 gv = ldf4(&sm.gpos[cb][r0]);
      f32x4 O;
#pragma unroll
      for (int i = 0; i < 4; ++i) O[i] = scale * gv[i] * QSr[i];
#pragma unroll
      for (int jp = 0; jp < 2; ++jp)
        if (jp == 0 || w4 >= 2)
          O = mfma32(pmf[jp], cat8(sm.U[2 * jp][l], sm.U[2 * jp + 1][l]), O);
      const float gC = sm.gpos[cb][FC - 1];
      h16x8 udb[2];
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) udb[jp] = cat8(sm.Ud[2 * jp][l], sm.Ud[2 * jp + 1][l]);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x4 acc = gC * S[hh];
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) acc = mfma32(ktf[hh][jp], udb[jp], acc);
        S[hh] = acc;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = cc * FC + r0 + i;
        if (t < T) oh[(size_t)t * v_tok + lr] = from_f32<TOut>(O[i]);
      }
    }
    __syncthreads();
  }
  if (state_out) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 32 * w4 + 16 * hh + 4 * lq + i;
        state_out[((size_t)bh * FDK + row) * DV + col0 + lr] = S[hh][i];
      }
    }
  }
}

}  // namespace

bool prefill_fused_supported(const PrefillArgs& p) {
  return p.bf16 && p.Dk == FDK && p.chunk == FC && p.Dv % 16 == 0 && p.T > 0;
}

hipError_t launch_prefill_fused(const PrefillArgs& p) {
  const int NC = (p.T + FC - 1) / FC;
  const int NS = p.Dv / 16;
  const int grid = p.B * p.H * NS;
  if (p.out_bf16) {
    hipLaunchKernelGGL(prefill_fused_kernel<bf16>, dim3(grid), dim3(NTHR), 0,
                       (hipStream_t)p.stream, (const bf16*)p.q, (const bf16*)p.k,
                       (const bf16*)p.v, p.alpha, p.beta, p.state_in, p.state_out,
                       (bf16*)p.out, p.T, p.H, p.Dv, NC, NS, p.scale);
  } else {
    hipLaunchKernelGGL(prefill_fused_kernel<float>, dim3(grid), dim3(NTHR), 0,
                       (hipStream_t)p.stream, (const bf16*)p.q, (const bf16*)p.k,
                       (const bf16*)p.v, p.alpha, p.beta, p.state_in, p.state_out,
                       (float*)p.out, p.T, p.H, p.Dv, NC, NS, p.scale);
  }
  return hipGetLastError();
}

}  // namespace gdn
