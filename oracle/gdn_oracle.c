/*
 * Plain CPU oracle for the Gated DeltaNet (GDN) token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct ground
 * truth that the GPU library is checked against.  Only the test suite, the
 * package smoke check and the benchmark's CPU-baseline leg load it.  It shares
 * no code, header, table or helper with the GPU library, and the GPU library
 * never calls it.
 *
 * Source text followed (web page "The Key to Going Linear: Analysis-Driven
 * Transformer Linearization", Kuzina, Whatmough, Ehteshami Bejnordi):
 *   - section 3.1.2: read-out y_t = q_t^T S_t, and the GDN state update
 *     S_t = (I - beta_t k_t k_t^T) G_t S_{t-1} + beta_t k_t v_t^T;
 *   - section 3.1 (first display): causal softmax attention with 1/sqrt(d);
 *   - section 4, "Adding Sliding Window Attention": the disjoint linear +
 *     sink/window softmax output;
 *   - section 4, "Adapting Q/K/V": short convolutions on q, k, v;
 *   - appendix B.1, "Assumption Checks": key normalisation k / (||k||_2 + eps).
 *
 * Readings taken where the page leaves a step open:
 *   - S is key-major, d_k x d_v, and the read-out is o_t = scale * S_t^T q_t
 *     taken AFTER token t has been written (the page's y_t = q_t^T S_t).
 *   - The write term printed as "beta_t k_t^T v_t" is the outer product
 *     beta_t k_t v_t^T (a d_k x d_v matrix).
 *   - The gate G_t is a scalar alpha_t per (token, head): G_t = alpha_t I.
 *     The page applies G_t first and the erase (I - beta k k^T) second; with a
 *     scalar gate the two orders agree, and this code follows the page's order.
 *     The channel-wise variant G_t = diag(alpha_t) (section 3.2's diag gates)
 *     keeps that order, where it does matter.
 *   - Sliding window: the window is the w most recent tokens including the
 *     current one, the sinks are the first s tokens, and the linear state holds
 *     exactly the tokens that are in neither set.  Sets overlapping at short t
 *     are merged (each token is counted once).
 *   - Short convolution: per channel, causal, kernel K, taps[c][K-1] multiplies
 *     the current token, zero history before the first token, no bias, then
 *     SiLU; optionally an L2 normalisation over groups of channels.
 *
 * Every routine is a direct loop over the definition: no chunking, no
 * blocking, no algebraic rewrite.  Arithmetic is in double precision (the
 * "_f64" entry points); gdn_oracle_recurrence_f32 repeats the recurrence in
 * single precision so the tests can bound the oracle's own rounding.
 *
 * Layouts (all row-major, contiguous):
 *   q, k      [B, T, H, Dk]       v, out   [B, T, H, Dv]
 *   alpha,beta[B, T, H]           state    [B, H, Dk, Dv]
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* GDN recurrence, token by token (section 3.1.2).                            */
/*                                                                           */
/* For every (b, h) independently:                                           */
/*   S <- alpha_t S                          (G_t S_{t-1}, scalar gate)       */
/*   S <- S - beta_t k_t (k_t^T S)           ((I - beta k k^T) applied)       */
/*   S <- S + beta_t k_t v_t^T               (write)                         */
/*   o_t = scale * S^T q_t                   (read after write)              */
/* erase = 0 drops the middle line: this is the test hook that turns the      */
/* update into plain gated accumulation (the page's GLA, section 3.2).       */
/* state_in may be NULL (zero initial state); state_out may be NULL.          */
/* ------------------------------------------------------------------------- */
#define GDN_RECURRENCE_BODY(real)                                               \
  {                                                                             \
    long BH = (long)B * H;                                                      \
    _Pragma("omp parallel for schedule(dynamic, 1)")                            \
    for (long bh = 0; bh < BH; ++bh) {                                          \
      long b = bh / H, h = bh % H;                                              \
      real* S = (real*)malloc(sizeof(real) * (size_t)Dk * Dv);                  \
      real* p = (real*)malloc(sizeof(real) * (size_t)Dv);                       \
      if (state_in)                                                             \
        for (long e = 0; e < (long)Dk * Dv; ++e)                                \
          S[e] = (real)state_in[bh * Dk * Dv + e];                              \
      else                                                                      \
        for (long e = 0; e < (long)Dk * Dv; ++e) S[e] = 0;                      \
      for (long t = 0; t < T; ++t) {                                            \
        long row = (b * T + t) * H + h;                                         \
        const double* qt = q + row * Dk;                                        \
        const double* kt = k + row * Dk;                                        \
        const double* vt = v + row * Dv;                                        \
        real a = (real)alpha[row], be = (real)beta[row];                        \
        for (long e = 0; e < (long)Dk * Dv; ++e) S[e] = a * S[e];               \
        if (erase) {                                                            \
          for (long j = 0; j < Dv; ++j) {                                       \
            real acc = 0;                                                       \
            for (long i = 0; i < Dk; ++i) acc += (real)kt[i] * S[i * Dv + j];   \
            p[j] = acc;                                                         \
          }                                                                     \
          for (long i = 0; i < Dk; ++i)                                         \
            for (long j = 0; j < Dv; ++j)                                       \
              S[i * Dv + j] -= be * (real)kt[i] * p[j];                         \
        }                                                                       \
        for (long i = 0; i < Dk; ++i)                                           \
          for (long j = 0; j < Dv; ++j)                                         \
            S[i * Dv + j] += be * (real)kt[i] * (real)vt[j];                    \
        for (long j = 0; j < Dv; ++j) {                                         \
          real acc = 0;                                                         \
          for (long i = 0; i < Dk; ++i) acc += S[i * Dv + j] * (real)qt[i];     \
          out[row * Dv + j] = (double)((real)scale * acc);                      \
        }                                                                       \
      }                                                                         \
      if (state_out)                                                            \
        for (long e = 0; e < (long)Dk * Dv; ++e)                                \
          state_out[bh * Dk * Dv + e] = (double)S[e];                           \
      free(S);                                                                  \
      free(p);                                                                  \
    }                                                                           \
  }

void gdn_oracle_recurrence_f64(const double* q, const double* k, const double* v,
                               const double* alpha, const double* beta,
                               const double* state_in, double* state_out,
                               double* out, int B, int T, int H, int Dk, int Dv,
                               double scale, int erase)
GDN_RECURRENCE_BODY(double)

/* Same recurrence with every operation rounded to float; inputs and outputs
 * are still passed as double arrays. */
void gdn_oracle_recurrence_f32(const double* q, const double* k, const double* v,
                               const double* alpha, const double* beta,
                               const double* state_in, double* state_out,
                               double* out, int B, int T, int H, int Dk, int Dv,
                               double scale, int erase)
GDN_RECURRENCE_BODY(float)

/* ------------------------------------------------------------------------- */
/* GDN recurrence with a channel-wise gate G_t = diag(alpha_t), alpha_t in    */
/* R^{Dk} per (token, head) (section 3.2: the gate as a product of            */
/* diag(alpha_j); the section 3.1.2 update with a diagonal G_t).  S is        */
/* key-major, so G_t scales the rows of S.  For every (b, h):                 */
/*   gate_first = 1 (the page's order, G_t before the erase):                 */
/*     S <- diag(alpha_t) S;  S <- S - beta_t k_t (k_t^T S);                  */
/*   gate_first = 0 (test hook: the erase before the gate):                   */
/*     S <- S - beta_t k_t (k_t^T S);  S <- diag(alpha_t) S;                  */
/*   then S <- S + beta_t k_t v_t^T and o_t = scale * S^T q_t.                */
/* alpha: [B, T, H, Dk]; the other layouts as above.                          */
/* ------------------------------------------------------------------------- */
void gdn_oracle_recurrence_chgate_f64(const double* q, const double* k, const double* v,
                                      const double* alpha, const double* beta,
                                      const double* state_in, double* state_out,
                                      double* out, int B, int T, int H, int Dk, int Dv,
                                      double scale, int gate_first) {
  long BH = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    long b = bh / H, h = bh % H;
    double* S = (double*)malloc(sizeof(double) * (size_t)Dk * Dv);
    double* p = (double*)malloc(sizeof(double) * (size_t)Dv);
    for (long e = 0; e < (long)Dk * Dv; ++e) S[e] = state_in ? state_in[bh * Dk * Dv + e] : 0.0;
    for (long t = 0; t < T; ++t) {
      long row = (b * T + t) * H + h;
      const double* qt = q + row * Dk;
      const double* kt = k + row * Dk;
      const double* vt = v + row * Dv;
      const double* at = alpha + row * Dk;
      double be = beta[row];
      for (int pass = 0; pass < 2; ++pass) {
        if ((pass == 0) == (gate_first != 0)) {
          for (long i = 0; i < Dk; ++i)
            for (long j = 0; j < Dv; ++j) S[i * Dv + j] *= at[i];
        } else {
          for (long j = 0; j < Dv; ++j) {
            double acc = 0;
            for (long i = 0; i < Dk; ++i) acc += kt[i] * S[i * Dv + j];
            p[j] = acc;
          }
          for (long i = 0; i < Dk; ++i)
            for (long j = 0; j < Dv; ++j) S[i * Dv + j] -= be * kt[i] * p[j];
        }
      }
      for (long i = 0; i < Dk; ++i)
        for (long j = 0; j < Dv; ++j) S[i * Dv + j] += be * kt[i] * vt[j];
      for (long j = 0; j < Dv; ++j) {
        double acc = 0;
        for (long i = 0; i < Dk; ++i) acc += S[i * Dv + j] * qt[i];
        out[row * Dv + j] = scale * acc;
      }
    }
    if (state_out)
      for (long e = 0; e < (long)Dk * Dv; ++e) state_out[bh * Dk * Dv + e] = S[e];
    free(S);
    free(p);
  }
}

/* ------------------------------------------------------------------------- */
/* Gated linear attention with a key-dependent gate (kGLA, section 3.2.2):    */
/*   y_t = sum_{i<=t} ( q_t^T [prod_{j=i+1}^{t} diag(alpha_j)                  */
/*                              (I - beta_j Diag(k_j o k_j))] k_i ) v_i,       */
/* taken as the state recurrence it unrolls from (every factor is diagonal,   */
/* so the product's order does not matter):                                    */
/*   S_t = diag(alpha_t o (1 - beta_t k_t o k_t)) S_{t-1} + k_t v_t^T,         */
/*   o_t = scale * S_t^T q_t   (read after the write, i = t included).         */
/* Readings: the printed sum has no step size on the write, so the write is   */
/* k_i v_i^T; the sum runs over i <= t (causal); alpha_j is a d_k-vector per  */
/* token (diag(alpha_j)); a state S_0 (state_in, or zero) enters as the first  */
/* term, decayed by every gate from token 1 on.                                */
/* alpha [B,T,H,Dk]; beta [B,T,H].                                            */
/* ------------------------------------------------------------------------- */
void gdn_oracle_kgla_f64(const double* q, const double* k, const double* v,
                         const double* alpha, const double* beta,
                         const double* state_in, double* state_out, double* out,
                         int B, int T, int H, int Dk, int Dv, double scale) {
  long BH = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    long b = bh / H, h = bh % H;
    double* S = (double*)malloc(sizeof(double) * (size_t)Dk * Dv);
    for (long e = 0; e < (long)Dk * Dv; ++e) S[e] = state_in ? state_in[bh * Dk * Dv + e] : 0.0;
    for (long t = 0; t < T; ++t) {
      long row = (b * T + t) * H + h;
      const double* qt = q + row * Dk;
      const double* kt = k + row * Dk;
      const double* vt = v + row * Dv;
      const double* at = alpha + row * Dk;
      double be = beta[row];
      for (long i = 0; i < Dk; ++i) {
        double g = at[i] * (1.0 - be * kt[i] * kt[i]);
        for (long j = 0; j < Dv; ++j) S[i * Dv + j] = g * S[i * Dv + j] + kt[i] * vt[j];
      }
      for (long j = 0; j < Dv; ++j) {
        double acc = 0;
        for (long i = 0; i < Dk; ++i) acc += S[i * Dv + j] * qt[i];
        out[row * Dv + j] = scale * acc;
      }
    }
    if (state_out)
      for (long e = 0; e < (long)Dk * Dv; ++e) state_out[bh * Dk * Dv + e] = S[e];
    free(S);
  }
}

/* ------------------------------------------------------------------------- */
/* Gradient of the GDN recurrence (section 3.1.2, scalar gate) by the adjoint */
/* of the token loop: with A_t = alpha_t (I - beta_t k_t k_t^T) (symmetric),  */
/* S_t = A_t S_{t-1} + beta_t k_t v_t^T and o_t = scale S_t^T q_t, the total  */
/* gradient G_t = dL/dS_t obeys                                               */
/*   G_t = scale q_t do_t^T + A_{t+1} G_{t+1},   G_T-1 includes dS_T,         */
/* and with P = S_{t-1}, p = P^T k_t, g = G_t^T k_t:                           */
/*   dq_t = scale S_t do_t                                                    */
/*   dv_t = beta_t g                                                          */
/*   dalpha_t = <G_t, P> - beta_t g.p                                         */
/*   dbeta_t  = g.(v_t - alpha_t p)                                           */
/*   dk_t = -alpha_t beta_t (G_t p + P g) + beta_t G_t v_t                    */
/*   dS0 = A_0 G_0.                                                           */
/* dstate_out may be NULL (no gradient into the final state).  The forward    */
/* states are recomputed and kept for the whole sequence (small cases only).  */
/* ------------------------------------------------------------------------- */
void gdn_oracle_recurrence_bwd_f64(const double* q, const double* k, const double* v,
                                   const double* alpha, const double* beta,
                                   const double* state_in, const double* dout,
                                   const double* dstate_out, double* dq, double* dk,
                                   double* dv, double* dalpha, double* dbeta,
                                   double* dstate_in, int B, int T, int H, int Dk, int Dv,
                                   double scale) {
  long BH = (long)B * H;
  long SZ = (long)Dk * Dv;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    long b = bh / H, h = bh % H;
    double* Ss = (double*)malloc(sizeof(double) * (size_t)(T + 1) * SZ);  /* S_{-1} .. S_{T-1} */
    double* G = (double*)malloc(sizeof(double) * (size_t)SZ);
    double* p = (double*)malloc(sizeof(double) * (size_t)Dv);
    double* g = (double*)malloc(sizeof(double) * (size_t)Dv);
    for (long e = 0; e < SZ; ++e) Ss[e] = state_in ? state_in[bh * SZ + e] : 0.0;
    for (long t = 0; t < T; ++t) {
      long row = (b * T + t) * H + h;
      const double* kt = k + row * Dk;
      const double* vt = v + row * Dv;
      const double* P = Ss + t * SZ;
      double* S = Ss + (t + 1) * SZ;
      double a = alpha[row], be = beta[row];
      for (long j = 0; j < Dv; ++j) {
        double acc = 0;
        for (long i = 0; i < Dk; ++i) acc += kt[i] * P[i * Dv + j];
        p[j] = acc;
      }
      for (long i = 0; i < Dk; ++i)
        for (long j = 0; j < Dv; ++j)
          S[i * Dv + j] = a * (P[i * Dv + j] - be * kt[i] * p[j]) + be * kt[i] * vt[j];
    }
    for (long e = 0; e < SZ; ++e) G[e] = dstate_out ? dstate_out[bh * SZ + e] : 0.0;
    for (long t = T - 1; t >= 0; --t) {
      long row = (b * T + t) * H + h;
      const double* qt = q + row * Dk;
      const double* kt = k + row * Dk;
      const double* vt = v + row * Dv;
      const double* dot = dout + row * Dv;
      const double* P = Ss + t * SZ;
      const double* S = Ss + (t + 1) * SZ;
      double a = alpha[row], be = beta[row];
      for (long i = 0; i < Dk; ++i)
        for (long j = 0; j < Dv; ++j) G[i * Dv + j] += scale * qt[i] * dot[j];
      for (long i = 0; i < Dk; ++i) {
        double acc = 0;
        for (long j = 0; j < Dv; ++j) acc += S[i * Dv + j] * dot[j];
        dq[row * Dk + i] = scale * acc;
      }
      for (long j = 0; j < Dv; ++j) {
        double ap = 0, ag = 0;
        for (long i = 0; i < Dk; ++i) {
          ap += kt[i] * P[i * Dv + j];
          ag += kt[i] * G[i * Dv + j];
        }
        p[j] = ap;
        g[j] = ag;
      }
      double gp = 0, gvp = 0, gP = 0;
      for (long j = 0; j < Dv; ++j) {
        gp += g[j] * p[j];
        gvp += g[j] * (vt[j] - a * p[j]);
        dv[row * Dv + j] = be * g[j];
      }
      for (long e = 0; e < SZ; ++e) gP += G[e] * P[e];
      dalpha[row] = gP - be * gp;
      dbeta[row] = gvp;
      for (long i = 0; i < Dk; ++i) {
        double Gp = 0, Pg = 0, Gv = 0;
        for (long j = 0; j < Dv; ++j) {
          Gp += G[i * Dv + j] * p[j];
          Pg += P[i * Dv + j] * g[j];
          Gv += G[i * Dv + j] * vt[j];
        }
        dk[row * Dk + i] = -a * be * (Gp + Pg) + be * Gv;
      }
      /* G_{t-1} part carried back: A_t G_t = a (G - be k g^T) */
      for (long i = 0; i < Dk; ++i)
        for (long j = 0; j < Dv; ++j) G[i * Dv + j] = a * (G[i * Dv + j] - be * kt[i] * g[j]);
    }
    for (long e = 0; e < SZ; ++e) dstate_in[bh * SZ + e] = G[e];
    free(Ss);
    free(G);
    free(p);
    free(g);
  }
}

/* ------------------------------------------------------------------------- */
/* Membership of token i (0-based) in the exact-attention set of step t       */
/* (0-based) with s sinks and a window of w tokens (section 4, sliding        */
/* window display): sinks are tokens 0..s-1, the window is t-w+1..t.          */
/* ------------------------------------------------------------------------- */
static int in_exact_set(long i, long t, long s, long w) {
  if (i > t) return 0;
  if (i < s) return 1;
  return i >= t - w + 1;
}

/* ------------------------------------------------------------------------- */
/* Sink + sliding-window softmax attention at positions t_begin..T-1 of a     */
/* sequence (section 3.1 softmax restricted to the set I of section 4).       */
/* q, k, v, out: [B, T, H, D].  logits = softmax_scale * q_t . k_i.           */
/* Rows of out before t_begin are left untouched.                            */
/* ------------------------------------------------------------------------- */
void gdn_oracle_swa_sink_f64(const double* q, const double* k, const double* v,
                             double* out, int B, int T, int H, int D,
                             int n_sink, int window, double softmax_scale,
                             int t_begin) {
  long NT = (long)T - t_begin;
  long BHT = (long)B * H * NT;
#pragma omp parallel for schedule(dynamic, 16)
  for (long idx = 0; idx < BHT; ++idx) {
    long b = idx / ((long)H * NT), rem = idx % ((long)H * NT);
    long h = rem / NT, t = t_begin + rem % NT;
    const double* qt = q + ((b * T + t) * H + h) * D;
    double* ot = out + ((b * T + t) * H + h) * D;
    double zmax = -INFINITY;
    for (long i = 0; i <= t; ++i) {
      if (!in_exact_set(i, t, n_sink, window)) continue;
      const double* ki = k + ((b * T + i) * H + h) * D;
      double z = 0;
      for (long d = 0; d < D; ++d) z += qt[d] * ki[d];
      z *= softmax_scale;
      if (z > zmax) zmax = z;
    }
    double den = 0;
    for (long d = 0; d < D; ++d) ot[d] = 0;
    for (long i = 0; i <= t; ++i) {
      if (!in_exact_set(i, t, n_sink, window)) continue;
      const double* ki = k + ((b * T + i) * H + h) * D;
      const double* vi = v + ((b * T + i) * H + h) * D;
      double z = 0;
      for (long d = 0; d < D; ++d) z += qt[d] * ki[d];
      double e = exp(z * softmax_scale - zmax);
      den += e;
      for (long d = 0; d < D; ++d) ot[d] += e * vi[d];
    }
    for (long d = 0; d < D; ++d) ot[d] /= den;
  }
}

/* ------------------------------------------------------------------------- */
/* Hybrid layer output (section 4): y_t = q_t^T S_{lin(t)} + y_t^swa, where   */
/* the linear state holds exactly the tokens outside the sinks and the        */
/* window.  At step t the token leaving the window, j = t - w, enters the     */
/* state (if it is not a sink), with its own alpha_j, beta_j, k_j, v_j; the   */
/* state is then read with q_t.  The linear read uses (ql, kl, vl, alpha,     */
/* beta); the softmax path uses (qs, ks, vs).  The state starts at zero.      */
/* ql, kl [B,T,H,Dk]; vl [B,T,H,Dv]; qs, ks, vs [B,T,H,Dv] (one head dim).   */
/* ------------------------------------------------------------------------- */
void gdn_oracle_hybrid_f64(const double* ql, const double* kl, const double* vl,
                           const double* alpha, const double* beta,
                           const double* qs, const double* ks, const double* vs,
                           double* out, int B, int T, int H, int Dk, int Dv,
                           int n_sink, int window, double lin_scale,
                           double softmax_scale) {
  long BH = (long)B * H;
  double* swa = (double*)malloc(sizeof(double) * (size_t)B * T * H * Dv);
  gdn_oracle_swa_sink_f64(qs, ks, vs, swa, B, T, H, Dv, n_sink, window,
                          softmax_scale, 0);
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    long b = bh / H, h = bh % H;
    double* S = (double*)calloc((size_t)Dk * Dv, sizeof(double));
    double* p = (double*)malloc(sizeof(double) * (size_t)Dv);
    for (long t = 0; t < T; ++t) {
      long j = t - window;
      if (j >= n_sink) {
        long rj = (b * T + j) * H + h;
        const double* kj = kl + rj * Dk;
        const double* vj = vl + rj * Dv;
        double a = alpha[rj], be = beta[rj];
        for (long e = 0; e < (long)Dk * Dv; ++e) S[e] *= a;
        for (long c = 0; c < Dv; ++c) {
          double acc = 0;
          for (long i = 0; i < Dk; ++i) acc += kj[i] * S[i * Dv + c];
          p[c] = acc;
        }
        for (long i = 0; i < Dk; ++i)
          for (long c = 0; c < Dv; ++c) S[i * Dv + c] -= be * kj[i] * p[c];
        for (long i = 0; i < Dk; ++i)
          for (long c = 0; c < Dv; ++c) S[i * Dv + c] += be * kj[i] * vj[c];
      }
      long rt = (b * T + t) * H + h;
      const double* qt = ql + rt * Dk;
      for (long c = 0; c < Dv; ++c) {
        double acc = 0;
        for (long i = 0; i < Dk; ++i) acc += S[i * Dv + c] * qt[i];
        out[rt * Dv + c] = lin_scale * acc + swa[rt * Dv + c];
      }
    }
    free(S);
    free(p);
  }
  free(swa);
}

/* ------------------------------------------------------------------------- */
/* Depthwise causal short convolution + SiLU (+ optional L2 normalisation)    */
/* (section 4 "Adapting Q/K/V"; normalisation as in appendix B.1).            */
/* x, y: [B, T, Ch]; taps: [Ch, K].                                           */
/*   a = sum_{j=0}^{K-1} taps[c][j] * x[t-K+1+j][c]   (x[<0] = 0)              */
/*   y = a * sigmoid(a)                                                       */
/* If group > 0, every run of `group` consecutive channels of a token is      */
/* divided by (its L2 norm + eps).                                            */
/* ------------------------------------------------------------------------- */
void gdn_oracle_short_conv_silu_f64(const double* x, const double* taps,
                                    double* y, int B, int T, int Ch, int K,
                                    int group, double eps) {
  long BT = (long)B * T;
#pragma omp parallel for schedule(static)
  for (long bt = 0; bt < BT; ++bt) {
    long b = bt / T, t = bt % T;
    double* yt = y + bt * Ch;
    for (long c = 0; c < Ch; ++c) {
      double a = 0;
      for (long j = 0; j < K; ++j) {
        long ts = t - K + 1 + j;
        if (ts < 0) continue;
        a += taps[c * K + j] * x[(b * T + ts) * Ch + c];
      }
      yt[c] = a / (1.0 + exp(-a));
    }
    if (group > 0) {
      for (long g0 = 0; g0 < Ch; g0 += group) {
        double ss = 0;
        for (long c = g0; c < g0 + group; ++c) ss += yt[c] * yt[c];
        double inv = 1.0 / (sqrt(ss) + eps);
        for (long c = g0; c < g0 + group; ++c) yt[c] *= inv;
      }
    }
  }
}

/* ------------------------------------------------------------------------- */
/* One decode step of the same convolution (section 4 "Adapting Q/K/V": the   */
/* causal convolution evaluated at one new token), from the K - 1 previous    */
/* inputs of each channel.                                                    */
/* x, y: [B, Ch]; state_in, state_out: [B, K-1, Ch], oldest row first.        */
/*   window = (state_in[0], ..., state_in[K-2], x)                            */
/*   a = sum_{j=0}^{K-1} taps[c][j] * window[j][c];  y = a * sigmoid(a)       */
/*   state_out = (state_in[1], ..., state_in[K-2], x)                         */
/* Optional group L2 normalisation as above.                                  */
/* ------------------------------------------------------------------------- */
void gdn_oracle_short_conv_step_f64(const double* x, const double* taps,
                                    const double* state_in, double* state_out,
                                    double* y, int B, int Ch, int K, int group,
                                    double eps) {
  const long H1 = K - 1;
  for (long b = 0; b < B; ++b) {
    const double* xb = x + b * Ch;
    const double* sb = state_in + b * H1 * Ch;
    double* ob = state_out + b * H1 * Ch;
    double* yb = y + b * Ch;
    for (long c = 0; c < Ch; ++c) {
      double a = 0;
      for (long j = 0; j < K; ++j) {
        double w = (j < H1) ? sb[j * Ch + c] : xb[c];
        a += taps[c * K + j] * w;
      }
      yb[c] = a / (1.0 + exp(-a));
    }
    if (group > 0) {
      for (long g0 = 0; g0 < Ch; g0 += group) {
        double ss = 0;
        for (long c = g0; c < g0 + group; ++c) ss += yb[c] * yb[c];
        double inv = 1.0 / (sqrt(ss) + eps);
        for (long c = g0; c < g0 + group; ++c) yb[c] *= inv;
      }
    }
    for (long j = 0; j < H1; ++j)
      for (long c = 0; c < Ch; ++c)
        ob[j * Ch + c] = (j + 1 < H1) ? sb[(j + 1) * Ch + c] : xb[c];
  }
}

int gdn_oracle_num_threads(void) {
  int n = 1;
#ifdef _OPENMP
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
#endif
  return n;
}
