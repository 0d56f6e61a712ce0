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
// Wave roles (wave-uniform; every wave passes the same barriers, two per
// chunk, and the loops of all roles run the same number of iterations):
//   wave 0 (SA)   the recurrence's critical path for its slice.  It carries all
//                 of S (128 x 16, f32) in eight MFMA accumulator tiles and per
//                 chunk computes X = K S, Y, U = Tm Y and the S update with no
//                 exchange inside the chunk.  The K^T operands of the update
//                 come from LDS transpose reads (ds_read_b64_tr_b16).
//   wave 1 (SB)   one chunk in arrears: Q S, the output tile, and the two
//                 off-diagonal levels of Tm (its diagonal 16x16 blocks come
//                 from the prep waves); S and U reach it through LDS.
//   waves 2..7    prep one chunk ahead: the Gram products K K^T and Q K^T of
//                 the next chunk (each wave a fixed set of 16x16 tiles), the
//                 gate scaling into A and Pm, and the diagonal blocks of Tm as
//                 (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8) (L strictly
//                 lower, L^16 = 0) with 16x16x16 MFMAs.  Waves 3, 5, 6, 7 also
//                 load the chunk after next from HBM (a two-deep register
//                 ring) and commit it to LDS as f16; wave 7 scans the gates.
// Per chunk c:
//   P1  SA: X_c, Y_c            SB: O_{c-1}, Tm levels of c   prep: Gram of c+1
//   P2  SA: U_c, S update       SB: Q_c S_c                   prep: A, Pm, diag Tm of c+1;
//                                                                   commit c+2, load c+4
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
// agree.  Lane group q = lane / 16 carries the indices {4q .. 4q+3} and
// {16 + 4q .. 16 + 4q + 3} of each 32-wide step, which is how two stacked
// accumulator tiles hold their rows: S, Y, U and the decayed U feed the next
// product straight from registers.  The K and Q tiles store their key columns
// permuted to match (within each group of 32, logical 16h + 4q + i sits at
// 8q + 4h + i), so those operands are single 16-byte reads; the Gram products
// contract over the permuted columns unchanged.
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
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

struct __align__(16) FusedSmem {
  h16 K[2][FC * FLD];      // K tiles of chunks (f16, [token][permuted key]), by parity
  h16 Q[2][FC * FLD];      // Q tiles
  f32x4 V[2][4][64];       // value slices, accumulator layout: [tile][lane][row]
  h16x8 Spub[2][4][64];    // S entering a chunk as B operands, per 32-key step
  h16x4 Upub[4][64];       // U of the last chunk, accumulator layout
  h16x4 Af[4][4][64];      // off-diagonal A blocks, A-operand layout
  h16x4 TDa[4][64];        // diagonal Tm blocks, A-operand layout
  h16x4 TDb[4][64];        // diagonal Tm blocks, accumulator layout
  h16x4 Tf[4][4][64];      // Tm, A-operand layout; upper blocks stay 0
  h16x4 Pmf[4][4][64];     // Pm, A-operand layout; upper blocks stay 0
  float gam[3][FC], gpos[3][FC], gneg[3][FC], bet[3][FC], dec[3][FC];  // by chunk % 3
  int wide[3];             // the chunk's log-gate range exceeds kWideGate
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
__device__ __forceinline__ h16x8 ld8(const h16* p) {
  return *reinterpret_cast<const h16x8*>(p);
}
// LDS transpose read: within each group of 16 lanes, lane i receives element
// (i & 3) of the 8-byte chunks addressed by lanes (i >> 2) + 4k, k = 0..3.
__device__ __forceinline__ h16x4 ld_tr(const h16* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(h16x4, r);
}
// Physical column of logical key column c in the K / Q tiles.
__device__ __forceinline__ int perm_col(int c) {
  return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}

// (I + L)^-1 and its transpose for a nilpotent 16x16 L (L^16 = 0), from L and
// L^T in accumulator layout (f32).  With M, M^T in accumulator layout,
// M N = mfma(M^T, N) and (M N)^T = mfma(N, M^T).
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
  int T, H, NC, NIT;
  float scale;
};

// Registers holding one chunk's share of the inputs for a commit thread.
struct ChunkRegs {
  bf16x8 k[4], q[4];
  bf16x4_t v;
  float a, b;
};

// Prep wave PW (0..5).  Gram tiles: row block RA (tiles (RA, 0..RA)) and, if
// RB >= 0, row block RB, of K K^T (GQ false) or Q K^T (GQ true):
//   PW 0: KK row 3        PW 1: QK row 3
//   PW 2: KK row 2        PW 3: QK rows 2, 0
//   PW 4: KK rows 1, 0    PW 5: QK row 1
// Commit threads CT (0..3): PW 1, 3, 4, 5; CT 3 also scans the gates.
template <int PW>
__device__ __forceinline__ void prep_loop(FusedSmem& sm, const PrepArgs& a, int l) {
  constexpr bool GQ = (PW & 1) != 0;
  constexpr int RA = (PW <= 1) ? 3 : (PW <= 3) ? 2 : 1;
  constexpr int RB = (PW == 3 || PW == 4) ? 0 : -1;
  constexpr int CT = (PW == 1) ? 0 : (PW == 3) ? 1 : (PW == 4) ? 2 : (PW == 5) ? 3 : -1;
  const int lr = l & 15, lq = l >> 4;
  const int T = a.T, NC = a.NC;
  const int pt = CT * 64 + l;  // commit thread 0..255 (meaningless if CT < 0)

  int off_qk[4] = {0, 0, 0, 0};
  int off_v = 0;
  if (CT >= 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int vi = pt + 256 * u;
      off_qk[u] = (vi >> 4) * (int)a.qk_tok + (vi & 15) * 8;
    }
    off_v = (pt >> 2) * (int)a.v_tok + (pt & 3) * 4;
  }
  ChunkRegs regs[2];

  auto prefetch = [&](int c, ChunkRegs& r) {
    const int t0 = c * FC;
    const bf16* kc = a.kh + (size_t)t0 * a.qk_tok;
    const bf16* qc = a.qh + (size_t)t0 * a.qk_tok;
    const bf16* vc = a.vh + (size_t)t0 * a.v_tok;
    if (t0 + FC <= T) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        r.k[u] = *reinterpret_cast<const bf16x8*>(kc + off_qk[u]);
        r.q[u] = *reinterpret_cast<const bf16x8*>(qc + off_qk[u]);
      }
      r.v = *reinterpret_cast<const bf16x4_t*>(vc + off_v);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (t0 + ((pt + 256 * u) >> 4) < T) {
          r.k[u] = *reinterpret_cast<const bf16x8*>(kc + off_qk[u]);
          r.q[u] = *reinterpret_cast<const bf16x8*>(qc + off_qk[u]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            r.k[u][e] = (bf16)0.f;
            r.q[u][e] = (bf16)0.f;
          }
        }
      }
      if (t0 + (pt >> 2) < T) {
        r.v = *reinterpret_cast<const bf16x4_t*>(vc + off_v);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) r.v[e] = (bf16)0.f;
      }
    }
    if (CT == 3) {
      const int t = t0 + l;
      r.a = (t < T) ? a.ah[(size_t)t * a.H] : 1.f;
      r.b = (t < T) ? a.bth[(size_t)t * a.H] : 0.f;
    }
  };

  // Registers -> LDS for chunk c: K, Q tiles as f16 (key columns permuted),
  // the value slice in accumulator layout, and (CT = 3) the gate tables.
  auto commit = [&](int c, const ChunkRegs& r) {
    const int nb = c & 1, g3 = c % 3;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int vi = pt + 256 * u;
      const int row = vi >> 4, c0 = (vi & 15) * 8;
      const int p0 = row * FLD + perm_col(c0), p1 = row * FLD + perm_col(c0 + 4);
      h16x4 k0, k1, q0, q1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k0[e] = (h16)(float)r.k[u][e];
        k1[e] = (h16)(float)r.k[u][4 + e];
        q0[e] = (h16)(float)r.q[u][e];
        q1[e] = (h16)(float)r.q[u][4 + e];
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
      for (int e = 0; e < 4; ++e) vb[(16 * qq + c4 + e) * 4 + ii] = (float)r.v[e];
    }
    if (CT == 3) {
      float la = logf(r.a);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(la, off);
        if (l >= off) la += y;
      }
      const float gl = __shfl(la, 63);
      const bool wide = gl < kWideGate;
      sm.gam[g3][l] = la;
      sm.gpos[g3][l] = __expf(la);
      sm.gneg[g3][l] = wide ? 0.f : __expf(-la);
      sm.bet[g3][l] = r.b;
      sm.dec[g3][l] = __expf(gl - la);
      if (l == 0) sm.wide[g3] = wide ? 1 : 0;
    }
  };

  // Gram accumulators.  Tile (R, Cb) is computed as mfma(K_Cb, X_R) with X = K
  // or Q: the result is (X K^T) restricted to the tile, in A-operand layout
  // (lane holds element (16R + lr, 16Cb + 4 lq + i)); for K K^T this uses its
  // symmetry.
  constexpr int NBB = (RB >= 0) ? RB + 1 : 1;
  f32x4 GA[RA + 1], GB[NBB];

  auto gram = [&](int c) {
    const int nb = c & 1;
    const h16* Kb = sm.K[nb];
    const h16* Qb = sm.Q[nb];
#pragma unroll
    for (int j = 0; j <= RA; ++j) GA[j] = zero4();
#pragma unroll
    for (int j = 0; j < NBB; ++j) GB[j] = zero4();
    for (int ks = 0; ks < 4; ++ks) {
      const int kc = ks * 32 + lq * 8;
      h16x8 kf[RA + 1];
#pragma unroll
      for (int cc = 0; cc <= RA; ++cc) kf[cc] = ld8(Kb + (16 * cc + lr) * FLD + kc);
      const h16x8 fa = GQ ? ld8(Qb + (16 * RA + lr) * FLD + kc) : kf[RA];
#pragma unroll
      for (int cc = 0; cc <= RA; ++cc) GA[cc] = mfma32(kf[cc], fa, GA[cc]);
      if (RB >= 0) {
        const h16x8 fb = GQ ? ld8(Qb + (16 * (RB < 0 ? 0 : RB) + lr) * FLD + kc)
                            : kf[RB < 0 ? 0 : RB];
#pragma unroll
        for (int cc = 0; cc < NBB; ++cc) GB[cc] = mfma32(kf[cc], fb, GB[cc]);
      }
    }
  };

  // Tile (R, Cb) -> Pm (QK waves), an off-diagonal block of A, or a diagonal
  // block of A whose inverse is written in both layouts.
  auto finish_tile = [&](int g3, bool wide, int R, int Cb, f32x4 G) {
    const float* gm = sm.gam[g3];
    const float* bt = sm.bet[g3];
    const int r = 16 * R + lr;        // this lane's row
    const int cb = 16 * Cb + 4 * lq;  // first of this lane's 4 columns
    const float rowf = GQ ? a.scale : bt[r];
    if (GQ || Cb < R) {
      f32x4 f;
      if (!wide) {
        const float rs = rowf * sm.gpos[g3][r];
        const f32x4 gn = ldf4(&sm.gneg[g3][cb]);
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
      for (int i = 0; i < 4; ++i) x[i] = (Cb < R || cb + i <= r) ? f[i] * G[i] : 0.f;
      if (GQ) {
        sm.Pmf[R][Cb][l] = cvt4(x);
      } else {
        sm.Af[R][Cb][l] = cvt4(x);
      }
    } else {
      // Diagonal block: G is symmetric, so lane (lq, lr) holds G at both
      // (4 lq + i, lr) and (lr, 4 lq + i).  L in accumulator layout takes
      // element (4 lq + i, lr); L^T takes element (lr, 4 lq + i) of L.
      const int rb = 16 * R;
      const f32x4 bv = ldf4(&bt[rb + 4 * lq]);
      f32x4 fL, fT;
      if (!wide) {
        const f32x4 gpv = ldf4(&sm.gpos[g3][rb + 4 * lq]);
        const f32x4 gnv = ldf4(&sm.gneg[g3][rb + 4 * lq]);
        const float gpl = sm.gpos[g3][rb + lr], gnl = sm.gneg[g3][rb + lr];
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
      sm.TDa[R][l] = cvt4(TTb);
      sm.TDb[R][l] = cvt4(Tb);
    }
  };

  auto finish = [&](int c) {
    const int g3 = c % 3;
    const bool wide = __builtin_amdgcn_readfirstlane(sm.wide[g3]) != 0;
#pragma unroll
    for (int cc = 0; cc <= RA; ++cc) finish_tile(g3, wide, RA, cc, GA[cc]);
    if (RB >= 0) {
#pragma unroll
      for (int cc = 0; cc < NBB; ++cc) finish_tile(g3, wide, RB < 0 ? 0 : RB, cc, GB[cc]);
    }
  };

  // One iteration of the common loop; R0 is the register set of chunk c + 2.
  auto iteration = [&](int c, ChunkRegs& r) {
    // P1: Gram of chunk c + 1.
    if (c + 1 >= 0 && c + 1 < NC) gram(c + 1);
    __syncthreads();
    // P2: A, Pm, diagonal Tm of chunk c + 1; commit chunk c + 2; load c + 4.
    if (c + 1 >= 0 && c + 1 < NC) finish(c + 1);
    if (CT >= 0) {
      if (c + 2 >= 0 && c + 2 < NC) commit(c + 2, r);
      if (c + 4 < NC) prefetch(c + 4, r);
    }
    __syncthreads();
  };

  if (CT >= 0) {
    if (0 < NC) prefetch(0, regs[0]);
    if (1 < NC) prefetch(1, regs[1]);
  }
  for (int it = 0; it < a.NIT; it += 2) {
    iteration(it - 2, regs[0]);
    iteration(it - 1, regs[1]);
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
  // Iterations c = -2 .. NC of the common loop, rounded up to an even count.
  const int NIT = (NC + 3 + 1) & ~1;

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

  if (wave >= 2) {
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
    pa.NIT = NIT;
    pa.scale = scale;
    switch (wave) {
      case 2: prep_loop<0>(sm, pa, l); break;
      case 3: prep_loop<1>(sm, pa, l); break;
      case 4: prep_loop<2>(sm, pa, l); break;
      case 5: prep_loop<3>(sm, pa, l); break;
      case 6: prep_loop<4>(sm, pa, l); break;
      default: prep_loop<5>(sm, pa, l); break;
    }
    return;
  }

  if (wave == 0) {
    // ============================ SA ============================
    // S tile m holds key rows 16m + 4 lq + i, value column col0 + lr.
    f32x4 S[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * m + 4 * lq + i;
        S[m][i] = state_in ? state_in[((size_t)bh * FDK + row) * DV + col0 + lr] : 0.f;
      }
    }
    // Transpose-read source chunk of this lane: key columns 16m + 4 (lr & 3)
    // .. +3 (contiguous after the permutation), token row offset lr >> 2.
    int kcolT[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) kcolT[m] = perm_col(16 * m + 4 * (lr & 3));
    const int trow = 4 * lq + (lr >> 2);

    h16x4 y16[4];
    h16x8 ktr[8][2];
    for (int it = 0; it < NIT; ++it) {
      const int c = it - 2;
      const bool run = c >= 0 && c < NC;
      const int b2 = c & 1, g3 = run ? c % 3 : 0;
      // P1: X = K S, Y = diag(beta) (V - diag(g) X); K^T operands of the update.
      if (run) {
        h16x8 sb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sb[j] = cat8(cvt4(S[2 * j]), cvt4(S[2 * j + 1]));
        const h16* Kb = sm.K[b2];
        const f32x4* Vb = &sm.V[b2][0][0];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          f32x4 X = zero4();
#pragma unroll
          for (int j = 0; j < 4; ++j)
            X = mfma32(ld8(Kb + (16 * rt + lr) * FLD + 32 * j + 8 * lq), sb[j], X);
          const int r0 = 16 * rt + 4 * lq;
          const f32x4 bv = ldf4(&sm.bet[g3][r0]);
          const f32x4 gv = ldf4(&sm.gpos[g3][r0]);
          const f32x4 Vv = Vb[rt * 64 + l];
          h16x4 y;
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = (h16)(bv[i] * (Vv[i] - gv[i] * X[i]));
          y16[rt] = y;
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
#pragma unroll
          for (int jp = 0; jp < 2; ++jp) {
            ktr[m][jp] = cat8(ld_tr(Kb + (32 * jp + trow) * FLD + kcolT[m]),
                              ld_tr(Kb + (32 * jp + 16 + trow) * FLD + kcolT[m]));
          }
        }
      }
      __syncthreads();
      // P2: U = Tm Y; S <- g_C S + K^T diag(dec) U; publish U and the new S.
      if (run) {
        h16x8 udb[2];
        h16x4 ud[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          f32x4 U = zero4();
#pragma unroll
          for (int jp = 0; jp < 2; ++jp) {
            if (jp == 0 || rt >= 2) {
              const h16x8 ta = cat8(sm.Tf[rt][2 * jp][l], sm.Tf[rt][2 * jp + 1][l]);
              U = mfma32(ta, cat8(y16[2 * jp], y16[2 * jp + 1]), U);
            }
          }
          const f32x4 dv = ldf4(&sm.dec[g3][16 * rt + 4 * lq]);
          h16x4 u16, d16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            u16[i] = (h16)U[i];
            d16[i] = (h16)(dv[i] * U[i]);
          }
          sm.Upub[rt][l] = u16;
          ud[rt] = d16;
        }
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) udb[jp] = cat8(ud[2 * jp], ud[2 * jp + 1]);
        const float gC = sm.gpos[g3][FC - 1];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          f32x4 acc = gC * S[m];
#pragma unroll
          for (int jp = 0; jp < 2; ++jp) acc = mfma32(ktr[m][jp], udb[jp], acc);
          S[m] = acc;
        }
      }
      if (run || c == -1) {
        // S entering chunk c + 1, as the B operands of Q S.
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sm.Spub[(c + 1) & 1][j][l] = cat8(cvt4(S[2 * j]), cvt4(S[2 * j + 1]));
      }
      __syncthreads();
    }
    if (state_out) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * m + 4 * lq + i;
          state_out[((size_t)bh * FDK + row) * DV + col0 + lr] = S[m][i];
        }
      }
    }
    return;
  }

  // ============================== SB ==============================
  TOut* oh = out + (size_t)b * T * v_tok + (size_t)h * DV + col0;
  f32x4 QS[4];
  f32x4 gp[4];
  h16x8 pma[4][2];
  h16x8 qa[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    QS[rt] = zero4();
    gp[rt] = zero4();
  }
  for (int it = 0; it < NIT; ++it) {
    const int c = it - 2;
    // P1: output of chunk c - 1; Tm of chunk c; operands of chunk c.
    if (c >= 1 && c <= NC) {
      const int cp = c - 1;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 O;
#pragma unroll
        for (int i = 0; i < 4; ++i) O[i] = scale * gp[rt][i] * QS[rt][i];
#pragma unroll
        for (int jp = 0; jp < 2; ++jp)
          if (jp == 0 || rt >= 2)
            O = mfma32(pma[rt][jp], cat8(sm.Upub[2 * jp][l], sm.Upub[2 * jp + 1][l]), O);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = cp * FC + 16 * rt + 4 * lq + i;
          if (t < T) oh[(size_t)t * v_tok + lr] = from_f32<TOut>(O[i]);
        }
      }
    }
    if (c >= 0 && c < NC) {
      // Tm levels (blocks in A-operand layout for SA; T_10 also in
      // accumulator layout as a right factor of level 2):
      //   T_10 = -T_11 A_10 T_00,   T_32 = -T_33 A_32 T_22,
      //   T_2j = -T_22 Z_2j,   T_3j = -(T_32 Z_2j + T_33 Z_3j),
      //   Z_mj = A_m0 T_0j + A_m1 T_1j.
      const h16x4 x10 = cvt4(mfma16(sm.Af[1][0][l], sm.TDb[0][l], zero4()));
      const h16x4 ta11 = sm.TDa[1][l];
      const h16x4 tb10 = cvt4(-mfma16(ta11, x10, zero4()));
      sm.Tf[1][0][l] = cvt4(-mfma16(x10, ta11, zero4()));
      const h16x4 x32 = cvt4(mfma16(sm.Af[3][2][l], sm.TDb[2][l], zero4()));
      const h16x4 ta32 = cvt4(-mfma16(x32, sm.TDa[3][l], zero4()));
      sm.Tf[3][2][l] = ta32;
      const h16x4 ta22 = sm.TDa[2][l], ta33 = sm.TDa[3][l];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x4 Z2, Z3;
        if (j == 0) {
          const h16x4 t00 = sm.TDb[0][l];
          Z2 = mfma16(sm.Af[2][1][l], tb10, mfma16(sm.Af[2][0][l], t00, zero4()));
          Z3 = mfma16(sm.Af[3][1][l], tb10, mfma16(sm.Af[3][0][l], t00, zero4()));
        } else {
          const h16x4 t11 = sm.TDb[1][l];
          Z2 = mfma16(sm.Af[2][1][l], t11, zero4());
          Z3 = mfma16(sm.Af[3][1][l], t11, zero4());
        }
        const h16x4 z2 = cvt4(Z2), z3 = cvt4(Z3);
        sm.Tf[2][j][l] = cvt4(-mfma16(z2, ta22, zero4()));
        sm.Tf[3][j][l] = cvt4(-(mfma16(z2, ta32, zero4()) + mfma16(z3, ta33, zero4())));
      }
#pragma unroll
      for (int I = 0; I < 4; ++I) sm.Tf[I][I][l] = sm.TDa[I][l];
      // Operands of chunk c kept for the next iterations.
      const int b2 = c & 1, g3 = c % 3;
      const h16* Qb = sm.Q[b2];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) qa[rt][j] = ld8(Qb + (16 * rt + lr) * FLD + 32 * j + 8 * lq);
#pragma unroll
        for (int jp = 0; jp < 2; ++jp)
          pma[rt][jp] = (jp == 0 || rt >= 2)
                            ? cat8(sm.Pmf[rt][2 * jp][l], sm.Pmf[rt][2 * jp + 1][l])
                            : h16x8{};
        gp[rt] = ldf4(&sm.gpos[g3][16 * rt + 4 * lq]);
      }
    }
    __syncthreads();
    // P2: Q S of chunk c.
    if (c >= 0 && c < NC) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma32(qa[rt][j], sm.Spub[c & 1][j][l], acc);
        QS[rt] = acc;
      }
    }
    __syncthreads();
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
