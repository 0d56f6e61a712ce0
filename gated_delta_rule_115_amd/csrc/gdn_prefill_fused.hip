// Single-pass chunked GDN prefill for gfx950: bf16 inputs, d_k = 128,
// chunks of 64 tokens, value dimension split into 16-column slices.
//
// Method: "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 3.1.2 (S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1}
// + beta_t k_t v_t^T, o_t = scale * S_t^T q_t), computed chunk by chunk with the
// exact WY/UT rewrite.  Within a chunk (gam_r = cumulative log gate, g_r =
// exp(gam_r), state S entering the chunk):
//   A_ri = beta_r exp(gam_r - gam_i) k_r.k_i  (i < r),   Tm = (I + A)^-1
//   Y = diag(beta) (V - diag(g) K S),   U = Tm Y
//   O = scale diag(g) Q S + Pm U,   Pm_ri = scale exp(gam_r - gam_i) q_r.k_i (i <= r)
//   S <- g_C S + K^T diag(exp(gam_C - gam)) U
//
// Gate factoring.  With a reference log gate gam_m (the midpoint of the
// chunk's range) and D = diag(exp(gam_m - gam)), I + A = D^-1 (I + A0) D with
// A0_ri = beta_r k_r.k_i, so Tm = D^-1 T0 D, T0 = (I + A0)^-1.  Writing
// Y~ = D Y and U^ = T0 Y~ (so U = D^-1 U^):
//   S <- g_C S + exp(gam_C - gam_m) K^T U^
//   O = scale diag(g) Q S + scale diag(exp(gam - gam_m)) P0 U^,  P0 = lower(Q K^T)
// The gates then touch only vectors, never the C x C matrices.  The factors
// are bounded by exp(range / 2), so this form is used when the chunk's
// log-gate range is at most kWideRange; wider chunks build A and Pm with one
// exp per element (D = I), which is the unfactored rewrite above.
//
// One work-group of 8 waves owns one (batch, head, 16-column value slice) and
// walks all chunks.  q, k, v, alpha, beta are read once and o is written once;
// nothing goes through a workspace.  The slices of one head sit on one XCD and
// share its L2 copy of the q/k tiles.
//
// Waves w and w + 4 share a SIMD; the roles are paired so that each SIMD
// carries a similar mix of MFMA and VALU work.
//
// Pipeline.  Every wave runs the same loop of iterations, one barrier each;
// each role works on a different chunk and hands results on through LDS ring
// slots (no role waits for another inside an iteration).  At iteration i:
//   CM  (waves 6, 7)  chunk i: K tile -> LDS as f16 (key columns permuted);
//                     global loads for chunk i + 2
//   KK  (waves 1, 5)  chunk i - 1: Gram blocks of K K^T for two block rows,
//                     scaled into A; diagonal blocks 0, 1 of Tm inverted as
//                     (I + L)^-1 = (I + L^8)(I + L^4)(I + L^2)(I - L)
//   LV  (wave 4)      chunk i - 2: diagonal blocks 2, 3 of Tm, then the
//                     off-diagonal blocks (block forward substitution);
//                     chunk i: gate tables and the scaled V slice
//   CH  (wave 0)      chunk i - 3: the recurrence for this slice: X = K S,
//                     Y~, U^ = T Y~, S update.  S (128 x 16, f32) lives in
//                     eight MFMA accumulator tiles for the whole sequence.
//   OUT (waves 2, 3)  chunk i - 3: Q rows of two block rows (own global loads,
//                     f16), their Q K^T blocks -> P; chunk i - 4: Q S, P U^ and
//                     the output rows, staged in LDS; wave 5 (KK) stores them
//                     at iteration i + 1.  (Vector-memory counters count stores
//                     too, so a wave that waits for its loads would otherwise
//                     also wait for its earlier stores.)
//
// Operand layouts.  A 16x16 MFMA result is held by lane l as rows 4 (l/16) ..
// +3 of column l % 16 (accumulator layout, written D(M)).  The A-operand
// fragment of M is D(M^T), the B-operand fragment is D(M), so
// D(M N) = mfma(D(M^T), D(N)) and D((M N)^T) = mfma(D(N), D(M^T)).  The 32-deep
// products take lane group q = l / 16 as the contraction indices
// {4q .. 4q+3} u {16 + 4q .. 16 + 4q + 3}: two stacked accumulator tiles form
// one operand, so S, Y~ and U^ feed the next product straight from registers.
// The K tile keeps its key columns permuted to match (within each 32, logical
// 16h + 4q + i sits at 8q + 4h + i), so K fragments are single 16-byte reads;
// Q fragments are loaded from HBM in that order.  K^T fragments come from LDS
// transpose reads (ds_read_b64_tr_b16).
//
// Precision: bf16 inputs convert to f16 exactly (unit-scale values); products
// take f16 operands with f32 accumulation; S is f32.
#include "gdn_f16ops.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

using namespace f16ops;

constexpr int FC = 64;          // tokens per chunk
constexpr int FDK = 128;        // key dimension
constexpr int FLD = FDK + 8;    // f16 row stride of the K tile (272 B)
constexpr int NTHR = 512;
constexpr float kWideRange = 10.f;  // log-gate range above which gates are per element
// Scaled value slice in LDS: element (token t, column n) of row tile rt sits at
// rt * VRT + n * VCS + (t % 16).  The padding makes both the per-token writes
// (64 lanes, one column) and the 16-byte reads of 4 consecutive tokens of one
// column (accumulator layout) free of bank conflicts.
constexpr int VCS = 20;            // column stride (floats)
constexpr int VRT = 16 * VCS + 16; // row-tile stride (floats)
// Output staging [column][token] with column stride OCS: the 16-byte writes of
// 4 tokens of one column and the per-token reads are free of bank conflicts.
constexpr int OCS = FC + 4;

// Per-chunk gate tables (one slot per chunk in flight).
struct GateSlot {
  float a[FC];    // Y~ = a V - b X
  float b[FC];
  float bet[FC];  // beta
  float gam[FC];  // cumulative log gate from the chunk start
  float og[FC];   // O = og (Q S) + of (P U^)
  float of[FC];
  float dec[FC];  // exp(gam_C - gam)
  float gC;       // exp(gam_C)
  float cS;       // S <- gC S + cS K^T (U^, or dec U^ for a wide chunk)
  int wide;       // gate ratios formed per element
  int pad;
};

struct __align__(16) Smem {
  h16 K[4][FC * FLD];     // K tiles (f16, permuted key columns), slot = chunk & 3
  float Vt[4][4 * VRT];   // a * V: [row tile][column][token] (see VRT), slot = chunk & 3
  float Ost[2][16 * OCS]; // output rows of a chunk, f32 [column][token], slot = chunk & 1
  h16x4 Ga[2][6][64];     // A blocks 10, 20, 21, 30, 31, 32 as A operands, slot = chunk & 1
  h16x4 Td[2][4][64];     // D(T00), D(T00^T), D(T11), D(T11^T)
  f32x4 Ld[2][4][64];     // D(L2), D(L2^T), D(L3), D(L3^T): diagonal blocks 2, 3 of A
  h16x8 Tc[2][6][64];     // Tm operands of the recurrence (row tile, 32-step pairs)
  h16x8 Sp[2][4][64];     // S entering a chunk as B operands, per 32-key step
  h16x4 Up[2][4][64];     // U^ of a chunk, accumulator layout
  GateSlot g[5];          // slot = chunk % 5
};

// Physical column of logical key column c in the K tile.
__device__ __forceinline__ int perm_col(int c) {
  return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}

struct Args {
  const bf16* qh;   // q of this (batch, head), token 0
  const bf16* kh;
  const bf16* vh;   // v of this (batch, head), token 0, first column of the slice
  const float* ah;  // alpha of this (batch, head), token 0 (stride H)
  const float* bh;
  const float* state_in;   // this (batch, head, slice) or null
  float* state_out;
  void* out;               // o of this (batch, head), first column of the slice
  int qk_tok, v_tok;       // elements between consecutive tokens
  int T, H, NC, NIT, DV;
  float scale;
};

// ---------------------------------------------------------------- CM --------
// K rows 32 W .. 32 W + 31 of chunk i -> LDS (f16, permuted columns).  Each
// lane moves 8 pieces of 8 consecutive keys; chunk i + 2 is loaded into the
// registers just freed.
__device__ void role_commit(Smem& sm, const Args& a, int l, int W) {
  bf16x8 raw[2][8];
  auto load = [&](int c, bf16x8* r) {
    const int t0 = c * FC;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int vi = l + 64 * u;
      const int row = 32 * W + (vi >> 4), c0 = (vi & 15) * 8;
      if (t0 + row < a.T) {
        r[u] = *reinterpret_cast<const bf16x8*>(a.kh + (size_t)(t0 + row) * a.qk_tok + c0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) r[u][e] = (bf16)0.f;
      }
    }
  };
  auto body = [&](int it, auto P) {
    constexpr int p = decltype(P)::value;  // it & 1
    if (it < a.NC) {
      h16* Kb = sm.K[it & 3];
      h16x4 kh[8][2];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        kh[u][0] = bf16_to_h4(__builtin_shufflevector(raw[p][u], raw[p][u], 0, 1, 2, 3));
        kh[u][1] = bf16_to_h4(__builtin_shufflevector(raw[p][u], raw[p][u], 4, 5, 6, 7));
      }
      if (it + 2 < a.NC) load(it + 2, raw[p]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int vi = l + 64 * u;
        const int row = 32 * W + (vi >> 4), c0 = (vi & 15) * 8;
        *reinterpret_cast<h16x4*>(Kb + row * FLD + perm_col(c0)) = kh[u][0];
        *reinterpret_cast<h16x4*>(Kb + row * FLD + perm_col(c0 + 4)) = kh[u][1];
      }
    }
    lds_barrier();
  };
  if (0 < a.NC) load(0, raw[0]);
  if (1 < a.NC) load(1, raw[1]);
  for (int it = 0; it < a.NIT; it += 2) {
    body(it, ic<0>());
    body(it + 1, ic<1>());
  }
}

// ---------------------------------------------------------------- KK --------
// Block rows RA < RB of chunk i - 1: W 0 -> rows 0, 3; W 1 -> rows 1, 2.
// Gram tile (R, C) = mfma(K_C, K_R) is the A-operand fragment of (K K^T)_RC.
template <int W, class TOut>
__device__ void role_kk(Smem& sm, const Args& a, int l) {
  constexpr int RA = W == 0 ? 0 : 1;
  constexpr int RB = W == 0 ? 3 : 2;
  const int lr = l & 15, lq = l >> 4;

  // Off-diagonal block (R, C) -> A-operand fragment of A_RC (lane row 16R + lr).
  auto offdiag = [&](const GateSlot& gs, bool wide, int R, int C, f32x4 G) -> h16x4 {
    const int r = 16 * R + lr;
    f32x4 x;
    if (!wide) {
      const float rf = gs.bet[r];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = rf * G[i];
    } else {
      const float rf = gs.bet[r], gr = gs.gam[r];
      const f32x4 gc = ldf4(&gs.gam[16 * C + 4 * lq]);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = rf * __expf(gr - gc[i]) * G[i];
    }
    return cvt4(x);
  };
  // Diagonal block R: D(L) and D(L^T) from the symmetric Gram tile.
  auto diag = [&](const GateSlot& gs, bool wide, int R, f32x4 G, f32x4& Lf, f32x4& LTf) {
    const int rb = 16 * R;
    const f32x4 bv = ldf4(&gs.bet[rb + 4 * lq]);
    const float bl = gs.bet[rb + lr];
    f32x4 fL, fT;
    if (!wide) {
      fL = bv;
#pragma unroll
      for (int i = 0; i < 4; ++i) fT[i] = bl;
    } else {
      const f32x4 gv = ldf4(&gs.gam[rb + 4 * lq]);
      const float gl = gs.gam[rb + lr];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fL[i] = bv[i] * __expf(gv[i] - gl);
        fT[i] = bl * __expf(gl - gv[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Lf[i] = (4 * lq + i > lr) ? fL[i] * G[i] : 0.f;
      LTf[i] = (lr > 4 * lq + i) ? fT[i] * G[i] : 0.f;
    }
  };

  for (int it = 0; it < a.NIT; ++it) {
    const int c = it - 1;
    if (c >= 0 && c < a.NC) {
      const h16* Kb = sm.K[c & 3];
      f32x4 GA[RA + 1], GB[RB + 1];
#pragma unroll
      for (int j = 0; j <= RA; ++j) GA[j] = zero4();
#pragma unroll
      for (int j = 0; j <= RB; ++j) GB[j] = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kc = ks * 32 + lq * 8;
        h16x8 kf[RB + 1];
#pragma unroll
        for (int C = 0; C <= RB; ++C) kf[C] = ld8(Kb + (16 * C + lr) * FLD + kc);
#pragma unroll
        for (int C = 0; C <= RA; ++C) GA[C] = mfma32(kf[C], kf[RA], GA[C]);
#pragma unroll
        for (int C = 0; C <= RB; ++C) GB[C] = mfma32(kf[C], kf[RB], GB[C]);
      }
      const GateSlot& gs = sm.g[c % 5];
      const bool wide = __builtin_amdgcn_readfirstlane(gs.wide) != 0;
      const int s = c & 1;
      if (W == 0) {
        // Rows 0 and 3: A30, A31, A32; T00 in both layouts, T33^T.
#pragma unroll
        for (int C = 0; C < 3; ++C) sm.Ga[s][3 + C][l] = offdiag(gs, wide, 3, C, GB[C]);
        f32x4 L0, LT0, L3, LT3, T00, TT00;
        diag(gs, wide, 3, GB[3], L3, LT3);
        sm.Ld[s][2][l] = L3;
        sm.Ld[s][3][l] = LT3;
        diag(gs, wide, 0, GA[0], L0, LT0);
        inv16<true, true>(L0, LT0, lr, lq, T00, TT00);
        sm.Td[s][0][l] = cvt4(T00);
        sm.Td[s][1][l] = cvt4(TT00);
      } else {
        // Rows 1 and 2: A10, A20, A21; T11 and T22 in both layouts.
        sm.Ga[s][0][l] = offdiag(gs, wide, 1, 0, GA[0]);
        sm.Ga[s][1][l] = offdiag(gs, wide, 2, 0, GB[0]);
        sm.Ga[s][2][l] = offdiag(gs, wide, 2, 1, GB[1]);
        f32x4 L1, LT1, L2, LT2, T11, TT11;
        diag(gs, wide, 2, GB[2], L2, LT2);
        sm.Ld[s][0][l] = L2;
        sm.Ld[s][1][l] = LT2;
        diag(gs, wide, 1, GA[1], L1, LT1);
        inv16<true, true>(L1, LT1, lr, lq, T11, TT11);
        sm.Td[s][2][l] = cvt4(T11);
        sm.Td[s][3][l] = cvt4(TT11);
      }
    }
    // W 1 also writes the output rows of chunk i - 5 (staged by the output
    // waves): this wave issues no global loads, so nothing ever waits for the
    // stores to complete.  Lane = token.
    const int cs = it - 5;
    if (W == 1 && cs >= 0 && cs < a.NC && cs * FC + l < a.T) {
      const float* ob = &sm.Ost[cs & 1][l];
      float o[16];
#pragma unroll
      for (int n = 0; n < 16; ++n) o[n] = ob[n * OCS];
      TOut* dst = reinterpret_cast<TOut*>(a.out) + (size_t)(cs * FC + l) * a.v_tok;
      if constexpr (sizeof(TOut) == 2) {
        bf16x8 v0, v1;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          v0[n] = (bf16)o[n];
          v1[n] = (bf16)o[8 + n];
        }
        *reinterpret_cast<bf16x8*>(dst) = v0;
        *reinterpret_cast<bf16x8*>(dst + 8) = v1;
      } else {
#pragma unroll
        for (int n = 0; n < 16; n += 4)
          *reinterpret_cast<f32x4*>(dst + n) = f32x4{o[n], o[n + 1], o[n + 2], o[n + 3]};
      }
    }
    lds_barrier();
  }
}

// ---------------------------------------------------------------- LV --------
// Off-diagonal blocks of Tm for chunk i - 2 (block forward substitution):
//   T10 = -T11 A10 T00,  T32 = -T33 A32 T22,
//   T2j = -T22 Z2j,  T3j = -(T32 Z2j + T33 Z3j),  Zmj = Am0 T0j + Am1 T1j;
// gate tables and the scaled value slice of chunk i (lane = token).
__device__ void role_lv(Smem& sm, const Args& a, int l) {
  const int lr = l & 15, lq = l >> 4;
  float ra[2], rb[2];
  bf16x8 rv[2][2];
  auto load = [&](int c, int p) {
    const int t = c * FC + l;
    if (t < a.T) {
      ra[p] = a.ah[(size_t)t * a.H];
      rb[p] = a.bh[(size_t)t * a.H];
      const bf16* vp = a.vh + (size_t)t * a.v_tok;
      rv[p][0] = *reinterpret_cast<const bf16x8*>(vp);
      rv[p][1] = *reinterpret_cast<const bf16x8*>(vp + 8);
    } else {
      ra[p] = 1.f;
      rb[p] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        rv[p][0][e] = (bf16)0.f;
        rv[p][1][e] = (bf16)0.f;
      }
    }
  };
  auto body = [&](int it, auto P) {
    constexpr int p = decltype(P)::value;  // it & 1
    const int c = it - 2;
    if (c >= 0 && c < a.NC) {
      const int s = c & 1;
      const h16x4 ga10 = sm.Ga[s][0][l], ga20 = sm.Ga[s][1][l], ga21 = sm.Ga[s][2][l];
      const h16x4 ga30 = sm.Ga[s][3][l], ga31 = sm.Ga[s][4][l], ga32 = sm.Ga[s][5][l];
      const h16x4 d00 = sm.Td[s][0][l], d00t = sm.Td[s][1][l];
      const h16x4 d11 = sm.Td[s][2][l], d11t = sm.Td[s][3][l];
      f32x4 T22, TT22, T33, TT33;
      inv16<true, true>(sm.Ld[s][0][l], sm.Ld[s][1][l], lr, lq, T22, TT22);
      inv16<false, true>(sm.Ld[s][2][l], sm.Ld[s][3][l], lr, lq, T33, TT33);
      const h16x4 d22 = cvt4(T22), d22t = cvt4(TT22);
      const h16x4 d33t = cvt4(TT33);
      const h16x4 x10 = cvt4(mfma16(ga10, d00, zero4()));    // D(A10 T00)
      const h16x4 t10t = cvt4(-mfma16(x10, d11t, zero4()));  // D(T10^T)
      const h16x4 t10 = cvt4(-mfma16(d11t, x10, zero4()));   // D(T10)
      const h16x4 x32 = cvt4(mfma16(ga32, d22, zero4()));    // D(A32 T22)
      const h16x4 t32t = cvt4(-mfma16(x32, d33t, zero4()));  // D(T32^T)
      const h16x8 d0010 = cat8(d00, t10);
      const h16x4 z20 = cvt4(mfma32(cat8(ga20, ga21), d0010, zero4()));
      const h16x4 z30 = cvt4(mfma32(cat8(ga30, ga31), d0010, zero4()));
      const h16x4 z21 = cvt4(mfma16(ga21, d11, zero4()));
      const h16x4 z31 = cvt4(mfma16(ga31, d11, zero4()));
      const h16x4 t20t = cvt4(-mfma16(z20, d22t, zero4()));
      const h16x4 t21t = cvt4(-mfma16(z21, d22t, zero4()));
      const h16x8 t3233 = cat8(t32t, d33t);
      const h16x4 t30t = cvt4(-mfma32(cat8(z20, z30), t3233, zero4()));
      const h16x4 t31t = cvt4(-mfma32(cat8(z21, z31), t3233, zero4()));
      const h16x4 zz = {0, 0, 0, 0};
      sm.Tc[s][0][l] = cat8(d00t, zz);
      sm.Tc[s][1][l] = cat8(t10t, d11t);
      sm.Tc[s][2][l] = cat8(t20t, t21t);
      sm.Tc[s][3][l] = cat8(d22t, zz);
      sm.Tc[s][4][l] = cat8(t30t, t31t);
      sm.Tc[s][5][l] = t3233;
    }
    if (it < a.NC) {
      GateSlot& gs = sm.g[it % 5];
      float vf[16];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        vf[n] = (float)rv[p][0][n];
        vf[8 + n] = (float)rv[p][1][n];
      }
      const float lalpha = __logf(ra[p]), bt = rb[p];
      if (it + 2 < a.NC) load(it + 2, p);
      const float la = wave_incl_sum(lalpha);
      const float g0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, la), 0));
      const float gl = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, la), 63));
      const bool wide = (g0 - gl) > kWideRange;
      const float gm = 0.5f * (g0 + gl);
      const float g = __expf(la);
      const float av = wide ? bt : bt * __expf(gm - la);
      gs.a[l] = av;
      gs.b[l] = av * g;
      gs.bet[l] = bt;
      gs.gam[l] = la;
      gs.og[l] = a.scale * g;
      gs.of[l] = wide ? 1.f : a.scale * __expf(la - gm);
      gs.dec[l] = __expf(gl - la);
      if (l == 0) {
        gs.gC = __expf(gl);
        gs.cS = wide ? 1.f : __expf(gl - gm);
        gs.wide = wide ? 1 : 0;
      }
      // a * V: token l, column n -> (l / 16) * VRT + n * VCS + l % 16.
      float* vb = &sm.Vt[it & 3][(l >> 4) * VRT + (l & 15)];
#pragma unroll
      for (int n = 0; n < 16; ++n) vb[n * VCS] = av * vf[n];
    }
    lds_barrier();
  };
  if (0 < a.NC) load(0, 0);
  if (1 < a.NC) load(1, 1);
  for (int it = 0; it < a.NIT; it += 2) {
    body(it, ic<0>());
    body(it + 1, ic<1>());
  }
}

// ---------------------------------------------------------------- CH --------
__device__ void role_chain(Smem& sm, const Args& a, int l) {
  const int lr = l & 15, lq = l >> 4;
  // S tile m: key rows 16m + 4 lq + i, value column lr of the slice.
  f32x4 S[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * m + 4 * lq + i;
      S[m][i] = a.state_in ? a.state_in[(size_t)row * a.DV + lr] : 0.f;
    }
  }
  // Transpose-read source of this lane: key columns 16m + 4 (lr & 3) .. +3
  // (contiguous after the permutation) of token row 4 lq + (lr >> 2).
  int kcolT[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) kcolT[m] = perm_col(16 * m + 4 * (lr & 3));
  const int trow = 4 * lq + (lr >> 2);

  for (int it = 0; it < a.NIT; ++it) {
    const int c = it - 3;
    if (c >= 0 && c < a.NC) {
      const int s = c & 1;
      const h16* Kb = sm.K[c & 3];
      const GateSlot& gs = sm.g[c % 5];
      const bool wide = __builtin_amdgcn_readfirstlane(gs.wide) != 0;
      h16x8 sb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sb[j] = cat8(cvt4(S[2 * j]), cvt4(S[2 * j + 1]));
        sm.Sp[s][j][l] = sb[j];
      }
      // X = K S, Y~ = a V - b X.
      h16x4 y16[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 X = zero4();
#pragma unroll
        for (int j = 0; j < 4; ++j)
          X = mfma32(ld8(Kb + (16 * rt + lr) * FLD + 32 * j + 8 * lq), sb[j], X);
        const f32x4 bv = ldf4(&gs.b[16 * rt + 4 * lq]);
        const f32x4 Vv = ldf4(&sm.Vt[c & 3][rt * VRT + lr * VCS + 4 * lq]);
        y16[rt] = cvt4(Vv - bv * X);
      }
      h16x8 ktr[8][2];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
          ktr[m][jp] = cat8(ld_tr(Kb + (32 * jp + trow) * FLD + kcolT[m]),
                            ld_tr(Kb + (32 * jp + 16 + trow) * FLD + kcolT[m]));
        }
      }
      // U^ = T Y~ (lower block triangle; upper halves of the pairs are zero).
      const h16x8 ylo = cat8(y16[0], y16[1]), yhi = cat8(y16[2], y16[3]);
      f32x4 U[4];
      U[0] = mfma32(sm.Tc[s][0][l], ylo, zero4());
      U[1] = mfma32(sm.Tc[s][1][l], ylo, zero4());
      U[2] = mfma32(sm.Tc[s][3][l], yhi, mfma32(sm.Tc[s][2][l], ylo, zero4()));
      U[3] = mfma32(sm.Tc[s][5][l], yhi, mfma32(sm.Tc[s][4][l], ylo, zero4()));
      h16x4 u16[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        u16[rt] = cvt4(U[rt]);
        sm.Up[s][rt][l] = u16[rt];
      }
      h16x8 udb[2];
      if (!wide) {
        udb[0] = cat8(u16[0], u16[1]);
        udb[1] = cat8(u16[2], u16[3]);
      } else {
        h16x4 d16[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) d16[rt] = cvt4(ldf4(&gs.dec[16 * rt + 4 * lq]) * U[rt]);
        udb[0] = cat8(d16[0], d16[1]);
        udb[1] = cat8(d16[2], d16[3]);
      }
      const float gC = gs.gC, cS = gs.cS;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const f32x4 dS = mfma32(ktr[m][1], udb[1], mfma32(ktr[m][0], udb[0], zero4()));
        S[m] = gC * S[m] + cS * dS;
      }
    }
    lds_barrier();
  }
  if (a.state_out) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * m + 4 * lq + i;
        a.state_out[(size_t)row * a.DV + lr] = S[m][i];
      }
    }
  }
}

// --------------------------------------------------------------- OUT --------
// Block rows RA, RB (W 0 -> 0, 3; W 1 -> 1, 2).  Iteration i: Q rows of chunk
// i - 3 as f16 operands, their Q K^T blocks (tile (R, C) = mfma(K_C, Q_R), the
// A-operand fragment of (Q K^T)_RC) -> P; Q S and P U^ of chunk i - 4 and its
// output rows.  Q of chunk c is loaded at iteration c + 1.
template <int W, class TOut>
__device__ void role_out(Smem& sm, const Args& a, int l) {
  constexpr int RA = W == 0 ? 0 : 1;
  constexpr int RB = W == 0 ? 3 : 2;
  const int lr = l & 15, lq = l >> 4;

  bf16x4 raw[2][2][4][2];  // [chunk parity][block][k step][half]
  h16x8 qh[2][2][4];       // [chunk parity][block][k step]
  h16x4 pf[2][2][4];       // [chunk parity][block][block column]

  auto load = [&](int c, int p) {
    const int t0 = c * FC;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int R = b == 0 ? RA : RB;
      const int t = t0 + 16 * R + lr;
      const bf16* qp = a.qh + (size_t)t * a.qk_tok + 4 * lq;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (t < a.T) {
          raw[p][b][j][0] = *reinterpret_cast<const bf16x4*>(qp + 32 * j);
          raw[p][b][j][1] = *reinterpret_cast<const bf16x4*>(qp + 32 * j + 16);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            raw[p][b][j][0][e] = (bf16)0.f;
            raw[p][b][j][1][e] = (bf16)0.f;
          }
        }
      }
    }
  };

  auto body = [&](int it, auto P) {
    constexpr int p = decltype(P)::value;  // parity of chunks it - 3 and it - 1
    constexpr int pp = p ^ 1;              // parity of chunk it - 4
    const int c = it - 3;
    if (c >= 0 && c < a.NC) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) qh[p][b][j] = cvt8(raw[p][b][j][0], raw[p][b][j][1]);
      if (it - 1 < a.NC) load(it - 1, p);
      const h16* Kb = sm.K[c & 3];
      f32x4 GA[RA + 1], GB[RB + 1];
#pragma unroll
      for (int j = 0; j <= RA; ++j) GA[j] = zero4();
#pragma unroll
      for (int j = 0; j <= RB; ++j) GB[j] = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kc = ks * 32 + lq * 8;
        h16x8 kf[RB + 1];
#pragma unroll
        for (int C = 0; C <= RB; ++C) kf[C] = ld8(Kb + (16 * C + lr) * FLD + kc);
#pragma unroll
        for (int C = 0; C <= RA; ++C) GA[C] = mfma32(kf[C], qh[p][0][ks], GA[C]);
#pragma unroll
        for (int C = 0; C <= RB; ++C) GB[C] = mfma32(kf[C], qh[p][1][ks], GB[C]);
      }
      const GateSlot& gs = sm.g[c % 5];
      const bool wide = __builtin_amdgcn_readfirstlane(gs.wide) != 0;
      auto mk = [&](int R, int C, f32x4 G) -> h16x4 {
        f32x4 x;
        if (!wide) {
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = (C < R || 4 * lq + i <= lr) ? G[i] : 0.f;
        } else {
          const float gr = gs.gam[16 * R + lr];
          const f32x4 gc = ldf4(&gs.gam[16 * C + 4 * lq]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            x[i] = (C < R || 4 * lq + i <= lr) ? a.scale * __expf(gr - gc[i]) * G[i] : 0.f;
        }
        return cvt4(x);
      };
      const h16x4 zz = {0, 0, 0, 0};
#pragma unroll
      for (int C = 0; C < 4; ++C) {
        pf[p][0][C] = C <= RA ? mk(RA, C, GA[C <= RA ? C : 0]) : zz;
        pf[p][1][C] = C <= RB ? mk(RB, C, GB[C <= RB ? C : 0]) : zz;
      }
    }
    if (c < 0 && it >= 1 && it - 1 < a.NC) load(it - 1, p);
    const int cp = it - 4;
    if (cp >= 0 && cp < a.NC) {
      const int s = cp & 1;
      const GateSlot& gs = sm.g[cp % 5];
      const h16x8 ulo = cat8(sm.Up[s][0][l], sm.Up[s][1][l]);
      const h16x8 uhi = cat8(sm.Up[s][2][l], sm.Up[s][3][l]);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int R = b == 0 ? RA : RB;
        f32x4 QS = zero4();
#pragma unroll
        for (int j = 0; j < 4; ++j) QS = mfma32(qh[pp][b][j], sm.Sp[s][j][l], QS);
        f32x4 PU = mfma32(cat8(pf[pp][b][0], pf[pp][b][1]), ulo, zero4());
        if (R >= 2) PU = mfma32(cat8(pf[pp][b][2], pf[pp][b][3]), uhi, PU);
        const f32x4 og = ldf4(&gs.og[16 * R + 4 * lq]);
        const f32x4 of = ldf4(&gs.of[16 * R + 4 * lq]);
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = og[i] * QS[i] + of[i] * PU[i];
        *reinterpret_cast<f32x4*>(&sm.Ost[cp & 1][lr * OCS + 16 * R + 4 * lq]) = o;
      }
    }
    lds_barrier();
  };
  // Iteration it works on chunk it - 3, of parity (it + 1) & 1; the loop starts
  // at it = 0 and is unrolled by two.
  for (int it = 0; it < a.NIT; it += 2) {
    body(it, ic<1>());
    body(it + 1, ic<0>());
  }
}

template <class TOut>
__global__ __launch_bounds__(NTHR) void prefill_fused_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* state_in,
    float* state_out, TOut* __restrict__ out, int T, int H, int DV, int NC, int NS, float scale) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;

  int bh, slice;
  xcd_group_map(blockIdx.x, gridDim.x / NS, NS, &bh, &slice);
  const int b = bh / H, h = bh % H;
  const int col0 = slice * 16;

  Args a;
  a.qk_tok = H * FDK;
  a.v_tok = H * DV;
  a.qh = q + (size_t)b * T * a.qk_tok + (size_t)h * FDK;
  a.kh = k + (size_t)b * T * a.qk_tok + (size_t)h * FDK;
  a.vh = v + (size_t)b * T * a.v_tok + (size_t)h * DV + col0;
  a.ah = alpha + (size_t)b * T * H + h;
  a.bh = beta + (size_t)b * T * H + h;
  a.state_in = state_in ? state_in + (size_t)bh * FDK * DV + col0 : nullptr;
  a.state_out = state_out ? state_out + (size_t)bh * FDK * DV + col0 : nullptr;
  a.out = out + (size_t)b * T * a.v_tok + (size_t)h * DV + col0;
  a.T = T;
  a.H = H;
  a.NC = NC;
  // Chunk c's last step (the store of its output rows) runs at iteration c + 5;
  // the count is rounded up to even for the two-way unrolled loops.
  a.NIT = (NC + 5 + 1) & ~1;
  a.DV = DV;
  a.scale = scale;

  switch (wave) {
    case 0: role_chain(sm, a, l); break;
    case 1: role_kk<0, TOut>(sm, a, l); break;
    case 2: role_out<0, TOut>(sm, a, l); break;
    case 3: role_out<1, TOut>(sm, a, l); break;
    case 4: role_lv(sm, a, l); break;
    case 5: role_kk<1, TOut>(sm, a, l); break;
    default: role_commit(sm, a, l, wave - 6); break;
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
