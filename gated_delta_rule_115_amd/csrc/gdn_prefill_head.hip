// Per-head chunked GDN prefill for gfx950: bf16 inputs, d_k = d_v = 128,
// chunks of 64 tokens, one work-group per (batch, head).
//
// Method: "The Key to Going Linear: Analysis-Driven Transformer
// Linearization", section 3.1.2 (S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1}
// + beta_t k_t v_t^T, o_t = scale * S_t^T q_t), computed chunk by chunk with the
// exact WY/UT rewrite.  Within a chunk (gam_r = cumulative log gate from the
// chunk start, g_r = exp(gam_r), S entering the chunk):
//   A_ri = beta_r exp(gam_r - gam_i) k_r.k_i  (i < r),   Tm = (I + A)^-1
//   Y = diag(beta) (V - diag(g) K S),   U = Tm Y
//   O = scale diag(g) Q S + Pm U,   Pm_ri = scale exp(gam_r - gam_i) q_r.k_i (i <= r)
//   S <- g_C S + K^T diag(exp(gam_C - gam)) U
// With the midpoint gam_m of the chunk's log-gate range and D = diag(exp(gam_m
// - gam)), Tm = D^-1 T0 D with T0 = (I + A0)^-1, A0_ri = beta_r k_r.k_i, so the
// gates reach only vectors:
//   Y~ = av V - bx X,  av = beta exp(gam_m - gam),  bx = beta exp(gam_m)
//   U^ = T0 Y~,  S <- g_C S + c_S K^T U^,  c_S = exp(gam_C - gam_m)
//   O = og (Q S) + of (P0 U^),  og = scale g,  of = scale exp(gam - gam_m)
// (P0 = lower(Q K^T)).  A chunk whose log-gate range exceeds kWide uses the
// unfactored form (gate ratios per element, D = I, c_S = 1, U weighted by
// exp(gam_C - gam) in the state update).
//
// The state is carried as S = sigma S~ with a per-chunk scalar sigma: the
// update S~ <- (g_C sigma / c_S) S~ + K^T U^ then accumulates straight into
// the MFMA tiles that hold S~ (no element-wise pass after the products), with
// sigma <- c_S; X = K S = sigma K S~ and Q S = sigma Q S~ fold sigma into
// bx and og.
//
// Work split.  One work-group of 8 waves per head and sequence segment (see
// below).  The state S~ (128 x 128, f32) lives in MFMA accumulator tiles,
// 16-column slices per wave, for the whole segment.  Everything that does not
// depend on S -- gates, Gram products, the triangular inverse, Q K^T -- is
// computed once per chunk and shared through LDS; a chunk moves through
// stages (tile to LDS, Gram blocks and diagonal inverses, Tm off-diagonal
// blocks, recurrence step) in successive iterations, so the stages of
// different chunks run side by side between two work-group barriers.  The
// diagonal 16 x 16 blocks of Tm are inverted by forward substitution in f32
// (rounded to f16 once formed); the off-diagonal blocks follow by block
// forward substitution.  Global loads are inline asm issued one or two iterations
// ahead of their use in a fixed order per iteration, so every wait is a
// fixed vmcnt and loads stay in flight across the loop back-edge.
//
// Operand layouts: see gdn_f16ops.h.  Contractions over the key index use, in
// each 32-key step j, lane group q = l / 16 for keys 32 j + 8 q .. + 7, so K
// and Q fragments are single 16-byte LDS reads; S~ tile m therefore holds
// key 32 (m / 2) + 8 (r / 4) + 4 (m % 2) + r % 4 in accumulator row r, so two
// stacked tiles form the B operand directly.  K^T and (av V) fragments come
// from LDS transpose reads.  Outputs are formed transposed, D((Q S)^T) =
// mfma(S operand, Q operand), so each lane holds 4 consecutive columns of one
// token and writes them with one store.
//
// LDS tiles (K, Q, av V: 64 x 128 f16) have 288-byte rows.  Measured on
// gfx950 with 8 waves per CU, this padding runs the 16-byte fragment reads at
// ~195 bytes per clock and the transpose reads at 128 (a 256-byte row runs
// the transpose reads at 41); every read offset is a lane base plus a
// constant.
//
// Ragged tails: rows past T load a copy of the last token and get alpha = 1,
// beta = 0, which makes them exact no-ops (their A rows, Y~ rows and U^ rows
// vanish); their output rows are not stored.
//
// Sequence segments.  One work-group per head leaves most of the chip idle
// when B * H is small, so the chunks of a head are split into P segments of
// L chunks.  A chunk maps the state entering it affinely, S -> M_c S + B_c,
// with M_c = g_C I - c_S K^T T0 diag(bx) K (the same recurrence with V = 0)
// and B_c the image of S = 0; a segment composes these maps.  Three passes:
//   transition pass  (work-group per head and segment s < P - 1): the
//                    recurrence run on M (from the identity, V = 0) and B
//                    (from 0) side by side -- wave w holds columns
//                    16 w .. 16 w + 15 of both, so each K fragment serves two
//                    products -- giving the segment's map M_s, B_s (f32,
//                    workspace); all waves share the per-chunk stages;
//   combine pass     (work-group per head and 16-column slice): S_0 = state
//                    in, S_{s+1} = M_s S_s + B_s (f32 products), the initial
//                    state of every segment (workspace);
//   output pass      (work-group per head and segment): the recurrence and
//                    the outputs of the segment from its initial state, the
//                    last segment writing the final state; waves 0-3 run the
//                    recurrence (two 16-column slices each), waves 4-7 do the
//                    loads, conversions and shared per-chunk stages.
// This is an exact rewrite of the same recurrence (composition of the affine
// chunk maps); each pass rounds like the single pass does.
//
// Precision: bf16 inputs convert to f16 exactly (unit-scale values); products
// take f16 operands with f32 accumulation; S~ is f32.
#include <algorithm>
#include <cmath>

#include "gdn_f16ops.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

using namespace f16ops;

constexpr int HC = 64;     // tokens per chunk
constexpr int HD = 128;    // key and value dimension
constexpr int HNT = 512;   // threads per work-group
constexpr int HRS = 144;   // f16 row stride of the LDS tiles (288 bytes)
constexpr float kWide = 10.f;  // log-gate range above which gates are per element

struct HGate {
  float bet[HC];  // beta
  float gam[HC];  // cumulative log gate from the chunk start
  float av[HC];   // Y~ = av V - bx X
  float bx[HC];
  float og[HC];   // O = og (Q S) + of (P U^)
  float of[HC];
  float dec[HC];  // exp(gam_C - gam), wide chunks
  float gC;       // exp(gam_C)
  float cS;       // exp(gam_C - gam_m), 1 for a wide chunk
  float gCc;      // gC / cS
  int wide;
};

struct __align__(16) HSmem {
  h16 K[3][HC * HRS];    // K tiles, slot = chunk % 3
  h16 Q[HC * HRS];       // Q tile of the chunk whose outputs are formed next
  h16 V[HC * HRS];       // av V of the chunk in the recurrence
  h16x8 Tc[2][6][64];    // Tm operands (see tm_offdiag), slot = chunk & 1
  h16x4 Ab[6][64];       // A10, A20, A21, A30, A31, A32 as A operands
  h16x4 Dg[7][64];       // D(T00), D(T00^T), D(T11), D(T11^T), D(T22), D(T22^T), D(T33^T)
  h16x4 Pb[6][64][2];    // P operands per (row tile, 32-token step); halves = block columns
  HGate g[3];            // slot = chunk % 3
  float Iv4[kInv4Scratch];  // diagonal blocks of A, column-major (helper wave 4)
  float tap[3][4 * HD];  // fused short conv: this head's taps of q, k, v, [tap][channel]
};

// Slot of P block (R, C) in Pb: row tile R, 32-token step C / 2.
__device__ __forceinline__ int pslot(int R, int C) {
  return R == 0 ? 0 : R == 1 ? 1 : 2 * (R - 1) + (C >> 1);
}

// Global loads of the streamed tiles and gates.  The compiler does not track
// these: the kernel waits for them itself with vm_wait, so the loads stay in
// flight across the loop back-edge (the compiler's own accounting falls back
// to waiting for every load there).
__device__ __forceinline__ void gld16(bf16x8& r, const bf16* p) {
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
}
__device__ __forceinline__ void gld4(float& r, const float* p) {
  asm volatile("global_load_dword %0, %1, off" : "=v"(r) : "v"(p) : "memory");
}
// Wait until at most N vector-memory operations are outstanding.  The
// registers a load wrote are tied to the wait, so no read of them is placed
// before it and they stay reserved until the data has arrived.
template <int N>
__device__ __forceinline__ void vm_wait(bf16x8 (&r)[2]) {
  asm volatile("s_waitcnt vmcnt(%2)" : "+v"(r[0]), "+v"(r[1]) : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void vm_wait(float& a, float& b) {
  asm volatile("s_waitcnt vmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N) : "memory");
}

// Four consecutive output columns of one token (byte offset `off`).
template <class TOut>
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t rs, int off, f32x4 o) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  if constexpr (sizeof(TOut) == 2) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)o[i];
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rs, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rs, off, 0, 0);
  }
}

// Short convolution fused into the tile loads (section 4, "Adapting Q/K/V"):
// the kernels then read the raw projections and apply, per channel,
//   y_t = SiLU(sum_{j<4} taps[c][j] x_{t-3+j}),  x_{<0} = 0,
// then, for q and k, y / (||y||_2 + eps) over the head's 128 channels, in f32,
// and round the result to f16 once, as the MFMA operand (never to bf16).  A
// loader thread owns rows 4 g .. 4 g + 3 of a chunk and channels pc .. pc + 7
// and loads those rows and the three before them (from the previous chunk or
// segment; zero before the sequence start), so its rows' convolution needs no
// data from other threads; the 16 lanes sharing g hold one token's 128
// channels and sum the squares for the norm.
struct ConvTaps {
  const float *q, *k, *v;  // [H * 128][4] each
  float eps;
};
struct ConvRows {
  bf16x8 r[7];  // rows 4 g - 3 .. 4 g + 3
};
// Loads of the rows of chunk start t0 (relative to the segment start; tabs0
// = absolute token of the segment start) for row group g: rows before the
// sequence start read the segment's first row (zeroed when used), rows past
// the end read the last row.
__device__ __forceinline__ void conv_issue(ConvRows& x, const bf16* base, int t0, int g, int pc,
                                           int Ts, int tabs0, int tok) {
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const int t = min(max(t0 + 4 * g - 3 + j, -tabs0), Ts - 1);
    gld16(x.r[j], base + (ptrdiff_t)t * tok + pc);
  }
}
// Sum over the 16 lanes of a DPP row (every lane receives it): quad swaps,
// then the half-row and row mirrors.
__device__ __forceinline__ float row_sum16(float x) {
  auto dpp = [](float v, auto ctrl) -> float {
    constexpr int C = decltype(ctrl)::value;
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), C, 0xf, 0xf, false));
  };
  x += dpp(x, ic<0xB1>());   // quad_perm [1, 0, 3, 2]
  x += dpp(x, ic<0x4E>());   // quad_perm [2, 3, 0, 1]
  x += dpp(x, ic<0x141>());  // row_half_mirror
  x += dpp(x, ic<0x140>());  // row_mirror
  return x;
}
// The taps are staged in LDS tap-major and multiplied by -log2(e), so the
// weighted sum is a' = -log2(e) a and 2^a' = e^-a feeds the sigmoid
// directly: the kernels form o' = a' / (1 + 2^a') = -log2(e) SiLU(a) and
// fold the constant into the per-row factor that follows (the norm's, or
// v's gate factor).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// The convolution and SiLU of the thread's 4 rows (o' above, f32), and per
// row the factor m that turns o' into the operand: with l2, -1 / (||o||_2 +
// eps) over the head's 128 channels (o = SiLU(a)); without, -ln 2.  tabs_r0:
// absolute token of row 4 g - 3; taps: this head's scaled [4][128] in LDS;
// edge (uniform over the wave): the chunk starts within 3 tokens of the
// sequence start, so some rows may lie before it and read as zero.
__device__ __forceinline__ void conv_rows(const ConvRows& x, const float* taps, int pc, int tabs_r0,
                                          bool edge, bool l2, float eps, float (&o)[4][8],
                                          float (&m)[4]) {
  bf16x8 r[7];
#pragma unroll
  for (int j = 0; j < 7; ++j) r[j] = x.r[j];
  if (edge) {
#pragma unroll
    for (int j = 0; j < 7; ++j)
      if (tabs_r0 + j < 0) r[j] = bf16x8{};
  }
  // taps[j][c] (tap-major): the 16 lanes of a row group read 16 different
  // 32-byte runs of one tap row.
  float w[8][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 lo = ldf4(taps + j * HD + pc), hi = ldf4(taps + j * HD + pc + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e][j] = lo[e], w[e + 4][j] = hi[e];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) a = __builtin_fmaf(w[e][j], (float)r[u + j][e], a);
      o[u][e] = a * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(a));
      ss = __builtin_fmaf(o[u][e], o[u][e], ss);
    }
    if (l2) {
      // ||o'|| = log2(e) ||o||, so eps scales by log2(e) too.
      ss = row_sum16(ss);
      m[u] = -__builtin_amdgcn_rcpf(__builtin_sqrtf(ss) + eps * kLog2e);
    } else {
      m[u] = -kLn2;
    }
  }
}
// The 4 rows m o' (times av[4 g + u] when given) to a tile in f16.
__device__ __forceinline__ void conv_store(h16* tile, const float (&o)[4][8], const float (&m)[4],
                                           int g, int pc, const float* av) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float a = av ? av[4 * g + u] * m[u] : m[u];
    h16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (h16)(a * o[u][e]);
    *reinterpret_cast<h16x8*>(tile + (4 * g + u) * HRS + pc) = y;
  }
}
// Waits for every load still in flight at the end of a pipelined loop, with
// the registers they write tied to the wait: the loads of the last
// iterations are never consumed, and without the tie the compiler would
// take those registers as free while the loads are still in flight.
__device__ __forceinline__ void vm_drain(bf16x8 (&r)[2][2]) {
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(r[0][0]), "+v"(r[0][1]), "+v"(r[1][0]), "+v"(r[1][1])::"memory");
}
__device__ __forceinline__ void vm_drain(bf16x8 (&r)[2][4]) {
  asm volatile("s_waitcnt vmcnt(0)"
               : "+v"(r[0][0]), "+v"(r[0][1]), "+v"(r[0][2]), "+v"(r[0][3]), "+v"(r[1][0]),
                 "+v"(r[1][1]), "+v"(r[1][2]), "+v"(r[1][3])::"memory");
}
__device__ __forceinline__ void vm_drain(float (&a)[2], float (&b)[2]) {
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1])::"memory");
}
// Waits for the loads of a ConvRows (the registers are tied to the wait).
template <int N>
__device__ __forceinline__ void vm_wait_rows(ConvRows& x) {
  asm volatile("s_waitcnt vmcnt(%7)"
               : "+v"(x.r[0]), "+v"(x.r[1]), "+v"(x.r[2]), "+v"(x.r[3]), "+v"(x.r[4]), "+v"(x.r[5]),
                 "+v"(x.r[6])
               : "n"(N)
               : "memory");
}

// Per-head workspace of the segment split: M_s, B_s (segments 0 .. P - 2) and
// the initial states of segments 1 .. P - 1, each 128 x 128 f32 [key][column].
struct SegWs {
  float* M;
  float* B;
  float* S;
  __device__ __host__ size_t at(int bh, int s, int P) const { return ((size_t)bh * (P - 1) + s) * HD * HD; }
};

// Chunk ranges of a head's segments.  Segment 0 has L0 chunks: its output
// pass runs beside the transition passes of segments 1 .. P - 2, which cost
// less per chunk, so it is made shorter to finish with them.  Segments 1 ..
// P - 1 have L chunks (the last one may have fewer).
struct SegGeom {
  int P, L0, L, NCT;
  __device__ __host__ int first(int s) const { return s == 0 ? 0 : L0 + (s - 1) * L; }
  __device__ __host__ int count(int s) const {
    const int left = NCT - first(s);
    return s == 0 ? L0 : (left < L ? left : L);
  }
};

// Gram-tile scalings (lane row 16 R + lr, columns 16 C + 4 lq + i).
// Off-diagonal block (R, C) of A as an A operand.
__device__ __forceinline__ h16x4 a_offdiag(const HGate& gs, bool wide, int R, int C, f32x4 G,
                                           int lr, int lq) {
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
}
// Block (R, C) of P (lower triangle of Q K^T; gate ratios and scale for a
// wide chunk) as an A operand.
__device__ __forceinline__ h16x4 p_block(const HGate& gs, bool wide, int R, int C, f32x4 G, int lr,
                                         int lq, float scale) {
  f32x4 x;
  if (!wide) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (C < R || 4 * lq + i <= lr) ? G[i] : 0.f;
  } else {
    const float gr = gs.gam[16 * R + lr];
    const f32x4 gc = ldf4(&gs.gam[16 * C + 4 * lq]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = (C < R || 4 * lq + i <= lr) ? scale * __expf(gr - gc[i]) * G[i] : 0.f;
  }
  return cvt4(x);
}
// Diagonal block R: D(L) and D(L^T) from the symmetric Gram tile.
__device__ __forceinline__ void a_diag(const HGate& gs, bool wide, int R, f32x4 G, int lr, int lq,
                                       f32x4& Lf, f32x4& LTf) {
  const int rb0 = 16 * R;
  const f32x4 bv = ldf4(&gs.bet[rb0 + 4 * lq]);
  const float bl = gs.bet[rb0 + lr];
  f32x4 fL, fT;
  if (!wide) {
    fL = bv;
#pragma unroll
    for (int i = 0; i < 4; ++i) fT[i] = bl;
  } else {
    const f32x4 gv = ldf4(&gs.gam[rb0 + 4 * lq]);
    const float gl = gs.gam[rb0 + lr];
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
}
// Gate tables of one chunk from alpha, beta of token l (one wave, lane = token).
__device__ __forceinline__ void gate_tables(HGate& gs, float alpha_l, float beta_l, bool valid,
                                            float scale, int l) {
  const float lal = valid ? __logf(alpha_l) : 0.f;
  const float bt = valid ? beta_l : 0.f;
  const float la = wave_incl_sum(lal);
  const float g0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, la), 0));
  const float gl = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, la), 63));
  const bool wide = (g0 - gl) > kWide;
  const float gm = 0.5f * (g0 + gl);
  const float g = __expf(la);
  const float av = wide ? bt : bt * __expf(gm - la);
  gs.bet[l] = bt;
  gs.gam[l] = la;
  gs.av[l] = av;
  gs.bx[l] = av * g;
  gs.og[l] = scale * g;
  gs.of[l] = wide ? 1.f : scale * __expf(la - gm);
  gs.dec[l] = __expf(gl - la);
  if (l == 0) {
    gs.gC = __expf(gl);
    gs.cS = wide ? 1.f : __expf(gl - gm);
    gs.gCc = wide ? gs.gC : __expf(gm);
    gs.wide = wide ? 1 : 0;
  }
}
// S~ tile m, accumulator row r: key kap(m, r).
__device__ __forceinline__ int kap(int m, int r) {
  return 32 * (m >> 1) + 8 * (r >> 2) + 4 * (m & 1) + (r & 3);
}

// LDS of the transition pass.  Each stage of a chunk runs one iteration after
// the stage it reads (one work-group barrier per iteration), so the K tiles
// and gate tables are read up to three iterations after they were written.
struct __align__(16) TSmem {
  h16 K[4][HC * HRS];    // K tiles, slot = chunk % 4
  h16 V[2][HC * HRS];    // av V, slot = chunk % 2
  h16x8 Tc[2][6][64];    // Tm operands (see tm_offdiag), slot = chunk % 2
  h16x4 Ab[2][6][64];    // A10, A20, A21, A30, A31, A32 as A operands, slot = chunk % 2
  h16x4 Dg[2][7][64];    // D(T00), D(T00^T), D(T11), D(T11^T), D(T22), D(T22^T), D(T33^T)
  HGate g[4];            // slot = chunk % 4
  float Iv[4][kInvScratch];  // inverse scratch of waves 0-3
  float tap[2][4 * HD];  // fused short conv: this head's taps of k, v, [tap][channel]
};

// Transition pass of one segment (chunks c0 .. c0 + NC - 1 of head (b, h)):
// its map S -> M_s S + B_s, from the recurrence run on M~ (from the identity,
// V = 0) and B~ (from 0) side by side; wave w holds columns 16 w .. 16 w + 15
// of both.  Iteration i (one work-group barrier at its end):
//   all waves  K of chunk i -> LDS; recurrence step of chunk i - 3 (X~ of both
//              states with shared K fragments, Y~, U^, state update); av V of
//              chunk i - 2 -> LDS
//   waves 0-3  diagonal block w of A for chunk i - 1, inverted
//   waves 4-5  off-diagonal blocks of A for chunk i - 1
//   wave 6     off-diagonal blocks of Tm for chunk i - 2
//   wave 7     gate tables of chunk i
// Every chunk of a transition segment lies inside the sequence (only the last
// segment can be ragged, and it has no transition).  B_s and M_s go to dstB
// and dstM (128 x 128 f32, [key][column]).
// With the fused convolution (CV), waves 0-3 load and convolve K at the top
// of the iteration and waves 4-7 V at its end; wave 7 also loads the gates.
template <bool CV>
__device__ __forceinline__ void transition_segment(TSmem& sm, const bf16* __restrict__ k,
                                                   const bf16* __restrict__ v,
                                                   const float* __restrict__ alpha,
                                                   const float* __restrict__ beta, float* dstB,
                                                   float* dstM, int b, int h, int T, int TS,
                                                   int H, int c0, int NC, const ConvTaps& ct) {
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lr = l & 15, lq = l >> 4;
  const int tok = H * HD;                // elements between consecutive tokens
  const size_t head0 = ((size_t)b * TS + (size_t)c0 * HC) * tok + (size_t)h * HD;
  const int Ts = T - c0 * HC;            // tokens from the segment start to the sequence end
  const bf16* kh = k + head0;
  const bf16* vh = v + head0;
  const float* ah = alpha + ((size_t)b * TS + (size_t)c0 * HC) * H + h;
  const float* bhp = beta + ((size_t)b * TS + (size_t)c0 * HC) * H + h;

  // Tile pieces of this thread: rows pr and pr + 32, 8 columns from pc.
  const int pr = tid >> 4, pc = (tid & 15) * 8;
  auto ld_tile = [&](const bf16* base, int c, bf16x8* r) {
    c = min(max(c, 0), NC - 1);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = min(c * HC + pr + 32 * u, Ts - 1);
      gld16(r[u], base + (size_t)t * tok + pc);
    }
  };
  float ra[2], rb[2];  // alpha, beta of token l (used by the gate wave)
  auto ld_gate = [&](int c, int p) {
    c = min(c, NC - 1);
    const int t = min(c * HC + l, Ts - 1);
    gld4(ra[p], ah + (size_t)t * H);
    gld4(rb[p], bhp + (size_t)t * H);
  };
  // The lane offsets pass through an empty asm once per iteration, so the
  // compiler folds the constant parts of every LDS address into the
  // instructions' offset fields instead of hoisting one register per address.
  auto lane_offset = [](int& x) { asm volatile("" : "+v"(x)); };
  int st_off = pr * HRS + pc;               // tile store offset (second piece 32 rows on)
  int fb = lr * HRS + 8 * lq;               // fragment: row lr, keys 32 j + 8 lq .. + 7
  int tb = (4 * lq + (lr >> 2)) * HRS + 8 * (lr & 3);       // K^T transpose reads
  int vb = (4 * lq + (lr >> 2)) * HRS + 16 * w + 4 * (lr & 3);  // av V transpose reads
  auto frag = [&](const h16* tile, int R, int j) { return ld8(tile + fb + 16 * R * HRS + 32 * j); };

  // B~ in S, M~ in SM; tile m holds keys kap(m, 4 lq + i) of column 16 w + lr.
  f32x4 S[8], SM[8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      S[m][i] = 0.f;
      SM[m][i] = kap(m, 4 * lq + i) == 16 * w + lr ? 1.f : 0.f;
    }
  float sig = 1.f;

  // Two register slots per stream (slot = iteration parity).  Iteration i
  // issues K of chunk i + 2 (2 loads), gates of chunk i + 2 (2), V of chunk i
  // (2), in this order, and consumes each two iterations later, when 10
  // later operations have been issued.
  bf16x8 kr[2][2], vr[2][2];
  // Fused convolution: the rows of one chunk in flight per wave, K on waves
  // 0-3 and V on waves 4-7.  Every wave requests its next rows at the top of
  // iteration i (K of chunk i + 1; V of chunk i - 2) -- one definition of the
  // rows' registers per iteration, outside any branch -- and the gates of
  // chunk i + 1 in its middle.  K waves convolve K of chunk i into LDS at the
  // top, before their recurrence step; V waves convolve av V of chunk i - 2
  // at the end, after theirs, so on each SIMD one wave's convolution runs
  // beside the other's matrix products.
  ConvRows xc;
  const int cg = (tid & 255) >> 4, cpc = (tid & 15) * 8, tabs0 = c0 * HC;
  const bf16* xbase = w < 4 ? kh : vh;
  auto cissue = [&](int c) {
    c = min(max(c, 0), NC - 1);
    conv_issue(xc, xbase, c * HC, cg, cpc, Ts, tabs0, tok);
  };
  auto cput = [&](const float* taps, bool l2, int c, h16* tile, const float* av) {
    float o[4][8], m[4];
    conv_rows(xc, taps, cpc, tabs0 + c * HC + 4 * cg - 3, tabs0 + c * HC < 3, l2, ct.eps, o, m);
    conv_store(tile, o, m, cg, cpc, av);
  };
  if constexpr (CV) {
    // This head's taps of k and v -> LDS.
    for (int i = tid; i < 2 * HD * 4; i += HNT) {
      const int e = i % (HD * 4);  // [channel][tap] in memory, [tap][channel] in LDS
      sm.tap[i / (HD * 4)][(e & 3) * HD + (e >> 2)] =
          -kLog2e * (i < HD * 4 ? ct.k : ct.v)[(size_t)h * HD * 4 + e];
    }
    lds_barrier();
    if (w < 4) cissue(0);
    ld_gate(0, 0);
  } else {
    ld_tile(kh, 0, kr[0]);
    ld_tile(kh, 1, kr[1]);
    ld_gate(0, 0);
    ld_gate(1, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  auto wait10 = [](bf16x8* r) {
    asm volatile("s_waitcnt vmcnt(10)" : "+v"(r[0]), "+v"(r[1])::"memory");
  };

  auto body = [&](int it, auto Par) {
    constexpr int p = decltype(Par)::value;  // it & 1
    const int c1 = it - 1, c2 = it - 2, c3 = it - 3;
    const bool h1 = c1 >= 0 && c1 < NC;
    const bool h2 = c2 >= 0 && c2 < NC;
    const bool h3 = c3 >= 0 && c3 < NC;
    lane_offset(st_off);
    lane_offset(fb);
    lane_offset(tb);
    lane_offset(vb);
    // Lane index, re-derived each iteration (keeps per-lane LDS addresses and
    // masks from being hoisted out of the loop as one register each).
    int ll = l;
    lane_offset(ll);
    const int llr = ll & 15, llq = ll >> 4;

    if constexpr (CV) {
      // K waves wait for K of chunk it here; for V waves, whose rows arrived
      // before the end of the previous iteration, the wait is already met.
      vm_wait_rows<2>(xc);
      if (w < 4 && it < NC) {
        // K of chunk it -> LDS (slot it % 4 was last read at iteration it - 1).
        cput(sm.tap[0], true, it, sm.K[it & 3], nullptr);
      }
      cissue(w < 4 ? it + 1 : it - 2);
    } else {
      wait10(kr[p]);
      if (it < NC) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
          *reinterpret_cast<h16x8*>(sm.K[it & 3] + st_off + 32 * u * HRS) = bf16x8_to_h8(kr[p][u]);
      }
      ld_tile(kh, it + 2, kr[p]);
    }

    auto recurrence = [&]() {
      if (h3) {
        // ---- recurrence step of chunk c3
        const h16* Kb = sm.K[c3 & 3];
        const HGate& gs = sm.g[c3 & 3];
        const bool wide = __builtin_amdgcn_readfirstlane(gs.wide) != 0;
        // X~ of B~ and of M~ share the K fragments.  Per 32-key step j: four K
        // fragments, the f16 state rows of that step, eight products; the
        // fragments of step j + 1 are requested during the products of step j.
        f32x4 X[4], XM[4];
  #pragma unroll
        for (int rt = 0; rt < 4; ++rt) X[rt] = zero4(), XM[rt] = zero4();
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          h16x8 kf[4];
  #pragma unroll
          for (int rt = 0; rt < 4; ++rt) kf[rt] = frag(Kb, rt, j);
          const h16x8 sb = cat8(cvt4(S[2 * j]), cvt4(S[2 * j + 1]));
          const h16x8 sm8 = cat8(cvt4(SM[2 * j]), cvt4(SM[2 * j + 1]));
  #pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            X[rt] = mfma32(kf[rt], sb, X[rt]);
            XM[rt] = mfma32(kf[rt], sm8, XM[rt]);
          }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  #pragma unroll
        for (int j = 0; j < 3; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        const float rho = gs.gCc * sig;
  #pragma unroll
        for (int m = 0; m < 8; ++m) S[m] *= rho, SM[m] *= rho;
        // av V, bx and Tm for Y~ and U^ and the first half of the K^T fragments
        // (keys 32 (m / 2) + 8 (lr % 4) + 4 (m % 2) .. + 3 of token rows
        // 4 lq + lr / 4 + 16 r) are requested ahead of the dependent chain.
        h16x4 va[4], kt[8][4];
        f32x4 bv[4];
        h16x8 tc[6];
  #pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          va[rt] = ld_tr(sm.V[c3 & 1] + vb + 16 * rt * HRS);
          bv[rt] = ldf4(&gs.bx[16 * rt + 4 * llq]);
        }
  #pragma unroll
        for (int i = 0; i < 6; ++i) tc[i] = sm.Tc[c3 & 1][i][ll];
        auto ktr = [&](int m, int r) { return ld_tr(Kb + tb + 16 * r * HRS + 32 * (m >> 1) + 4 * (m & 1)); };
  #pragma unroll
        for (int m = 0; m < 8; ++m) kt[m][0] = ktr(m, 0), kt[m][1] = ktr(m, 1);
        __builtin_amdgcn_sched_barrier(0);
        // U^ = T0 Y~ with Y~ = av V - (bx sigma) X~ (accumulator layout: tokens
        // 16 rt + 4 lq + i, column lr), for B~ (with V) and M~ (V = 0).  Returns
        // U^ weighted for the state update (by exp(gam_C - gam) for a wide chunk).
        auto solve = [&](const f32x4* Xs, bool withv, h16x8* udb) {
          h16x4 y16[4];
  #pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            f32x4 y;
  #pragma unroll
            for (int i = 0; i < 4; ++i)
              y[i] = (withv ? (float)va[rt][i] : 0.f) - (bv[rt][i] * sig) * Xs[rt][i];
            y16[rt] = cvt4(y);
          }
          const h16x8 ylo = cat8(y16[0], y16[1]), yhi = cat8(y16[2], y16[3]);
          f32x4 U[4];
          U[0] = mfma32(tc[0], ylo, zero4());
          U[1] = mfma32(tc[1], ylo, zero4());
          U[2] = mfma32(tc[2], ylo, zero4());
          U[3] = mfma32(tc[4], ylo, zero4());
          U[2] = mfma32(tc[3], yhi, U[2]);
          U[3] = mfma32(tc[5], yhi, U[3]);
          h16x4 u16[4];
          if (!wide) {
  #pragma unroll
            for (int rt = 0; rt < 4; ++rt) u16[rt] = cvt4(U[rt]);
          } else {
  #pragma unroll
            for (int rt = 0; rt < 4; ++rt) u16[rt] = cvt4(ldf4(&gs.dec[16 * rt + 4 * llq]) * U[rt]);
          }
          udb[0] = cat8(u16[0], u16[1]);
          udb[1] = cat8(u16[2], u16[3]);
        };
        h16x8 udb[2], udbm[2];
        solve(X, true, udb);
        solve(XM, false, udbm);
  #pragma unroll
        for (int m = 0; m < 8; ++m) kt[m][2] = ktr(m, 2), kt[m][3] = ktr(m, 3);
        __builtin_amdgcn_sched_barrier(0);
        // S~ += K^T U^, breadth-first over the sixteen state tiles.
  #pragma unroll
        for (int m = 0; m < 8; ++m) {
          const h16x8 k0 = cat8(kt[m][0], kt[m][1]);
          S[m] = mfma32(k0, udb[0], S[m]);
          SM[m] = mfma32(k0, udbm[0], SM[m]);
        }
  #pragma unroll
        for (int m = 0; m < 8; ++m) {
          const h16x8 k1 = cat8(kt[m][2], kt[m][3]);
          S[m] = mfma32(k1, udb[1], S[m]);
          SM[m] = mfma32(k1, udbm[1], SM[m]);
        }
        sig = gs.cS;
      }
    };
    auto shared_stage = [&]() {
      if (w < 4) {
        if (h1) {
          // Diagonal block R = w of A for chunk c1, inverted.
          const h16* Kb = sm.K[c1 & 3];
          const HGate& gs = sm.g[c1 & 3];
          const bool wide = __builtin_amdgcn_readfirstlane(gs.wide) != 0;
          f32x4 G = zero4();
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const h16x8 kf = frag(Kb, w, j);
            G = mfma32(kf, kf, G);
          }
          f32x4 Lb, LT, Tt, TT;
          a_diag(gs, wide, w, G, llr, llq, Lb, LT);
          inv16(LT, llr, llq, sm.Iv[w], Tt, TT);
          if (w < 3) {
            sm.Dg[c1 & 1][2 * w][ll] = cvt4(Tt);
            sm.Dg[c1 & 1][2 * w + 1][ll] = cvt4(TT);
          } else {
            sm.Dg[c1 & 1][6][ll] = cvt4(TT);
          }
        }
      } else if (w < 6) {
        if (h1) {
          // Off-diagonal blocks of A for chunk c1: rows 1, 2 (wave 4) or 3 (wave 5).
          const h16* Kb = sm.K[c1 & 3];
          const HGate& gs = sm.g[c1 & 3];
          const bool wide = __builtin_amdgcn_readfirstlane(gs.wide) != 0;
          h16x4* ab = sm.Ab[c1 & 1][0];
          f32x4 G0 = zero4(), G1 = zero4(), G2 = zero4();
          if (w == 4) {
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              const h16x8 k0 = frag(Kb, 0, j), k1 = frag(Kb, 1, j), k2 = frag(Kb, 2, j);
              G0 = mfma32(k0, k1, G0);  // (1, 0)
              G1 = mfma32(k0, k2, G1);  // (2, 0)
              G2 = mfma32(k1, k2, G2);  // (2, 1)
            }
            ab[0 * 64 + ll] = a_offdiag(gs, wide, 1, 0, G0, llr, llq);
            ab[1 * 64 + ll] = a_offdiag(gs, wide, 2, 0, G1, llr, llq);
            ab[2 * 64 + ll] = a_offdiag(gs, wide, 2, 1, G2, llr, llq);
          } else {
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              const h16x8 k3 = frag(Kb, 3, j);
              G0 = mfma32(frag(Kb, 0, j), k3, G0);  // (3, 0)
              G1 = mfma32(frag(Kb, 1, j), k3, G1);  // (3, 1)
              G2 = mfma32(frag(Kb, 2, j), k3, G2);  // (3, 2)
            }
            ab[3 * 64 + ll] = a_offdiag(gs, wide, 3, 0, G0, llr, llq);
            ab[4 * 64 + ll] = a_offdiag(gs, wide, 3, 1, G1, llr, llq);
            ab[5 * 64 + ll] = a_offdiag(gs, wide, 3, 2, G2, llr, llq);
          }
        }
      } else if (w == 6) {
        if (h2) {
          // Off-diagonal blocks of Tm for chunk c2 (block forward substitution).
          h16x4 ga[6], d[7];
          h16x8 tc[6];
  #pragma unroll
          for (int i = 0; i < 6; ++i) ga[i] = sm.Ab[c2 & 1][i][ll];
  #pragma unroll
          for (int i = 0; i < 7; ++i) d[i] = sm.Dg[c2 & 1][i][ll];
          tm_offdiag(ga, d, tc);
  #pragma unroll
          for (int i = 0; i < 6; ++i) sm.Tc[c2 & 1][i][ll] = tc[i];
        }
      }
    };
    recurrence();
    shared_stage();

    if constexpr (CV) {
      asm volatile("s_waitcnt vmcnt(7)" : "+v"(ra[0]), "+v"(rb[0])::"memory");
      if (w == 7 && it < NC) gate_tables(sm.g[it & 3], ra[0], rb[0], it * HC + ll < Ts, 1.f, ll);
      ld_gate(it + 1, 0);
      if (w >= 4) {
        // av V of chunk c2 -> LDS (slot c2 % 2 was last read at iteration
        // c2 + 1; the recurrence reads it at c2 + 3).
        vm_wait_rows<2>(xc);
        if (h2) cput(sm.tap[1], false, c2, sm.V[c2 & 1], sm.g[c2 & 3].av);
      }
      lds_barrier();
      return;
    }
    asm volatile("s_waitcnt vmcnt(10)" : "+v"(ra[p]), "+v"(rb[p])::"memory");
    if (w == 7 && it < NC) gate_tables(sm.g[it & 3], ra[p], rb[p], it * HC + ll < Ts, 1.f, ll);
    ld_gate(it + 2, p);

    wait10(vr[p]);
    if (h2) {
      // av V of chunk c2 -> LDS (its V tile was loaded at iteration c2).
      const HGate& gs = sm.g[c2 & 3];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float a = gs.av[pr + 32 * u];
        h16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (h16)(a * (float)vr[p][u][e]);
        *reinterpret_cast<h16x8*>(sm.V[c2 & 1] + st_off + 32 * u * HRS) = x;
      }
    }
    ld_tile(vh, it, vr[p]);
    lds_barrier();
  };

  // Chunk c completes its recurrence step at iteration c + 3.
  // The odd last iteration is peeled rather than guarded inside the loop, so
  // every path back to the loop head passes both copies of the body (the
  // fixed vmcnt waits count the loads of both).
  const int NIT = NC + 3;
  int it = 0;
  for (; it + 1 < NIT; it += 2) {
    body(it, ic<0>());
    body(it + 1, ic<1>());
  }
  if (it < NIT) body(it, ic<0>());
  if constexpr (CV) {
    vm_wait_rows<0>(xc);
  } else {
    vm_drain(kr);
    vm_drain(vr);
  }
  vm_drain(ra, rb);

  float* dst = dstB;
  float* dstm = dstM;
  // Recomputed here rather than kept live from the state set-up.
  int lq4 = 4 * lq, col = 16 * w + lr;
  lane_offset(lq4);
  lane_offset(col);
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = kap(m, lq4 + i) * HD + col;
      dst[o] = sig * S[m][i];
      dstm[o] = sig * SM[m][i];
    }
}

// Output pass of one segment (chunks c0 .. c0 + NC - 1 of head (b, h)) from
// the initial state s0 (null: zero), writing the final state to s_final
// unless null.  Wave roles: waves 0-3
// each run the recurrence of two 16-column slices (columns 32 c .. 32 c + 31),
// so every K, Q and K^T fragment read from LDS serves two products; waves
// 4-7 (one per SIMD, next to a recurrence wave) do all global loads, the
// f16 conversions, the Gram blocks, the inverse and the gate tables.
// Iteration i, phase 1: recurrence waves X~, (Q S~)^T, Y~ and U^ of chunk
// i - 2, and from the same K fragments the blocks (c, 0), (c, 1) of P (i - 2)
// for their wave c; helpers: K of chunk i -> LDS, the diagonal blocks of A
// and their inverses (chunk i - 1, all on helper 0), the off-diagonal blocks
// of A (i - 1), blocks (2, 2), (3, 2), (3, 3) of P (i - 2).  Phase 2:
// recurrence waves S~ update, (P U^)^T and the outputs of chunk i - 2;
// helpers: off-diagonal blocks of Tm (i - 1), gate tables (i), Q of chunk
// i - 1 and av V of chunk i - 1 -> LDS.
template <class TOut, bool CV>
__device__ __forceinline__ void out_segment(HSmem& sm, const bf16* __restrict__ q,
                                            const bf16* __restrict__ k,
                                            const bf16* __restrict__ v,
                                            const float* __restrict__ alpha,
                                            const float* __restrict__ beta, const float* s0,
                                            float* s_final, TOut* __restrict__ out, int b, int h,
                                            int T, int TS, int H, int c0, int NC, float scale,
                                            const ConvTaps& ct) {
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lr = l & 15, lq = l >> 4;
  const int tok = H * HD;                // elements between consecutive tokens
  const size_t head0 = ((size_t)b * TS + (size_t)c0 * HC) * tok + (size_t)h * HD;
  const int Ts = T - c0 * HC;            // tokens from the segment start to the sequence end
  const int NIT = NC + 2;                // chunk c's outputs are formed at iteration c + 2

  if (tid < 64) {  // zero halves of the P operands (block columns above the diagonal)
    sm.Pb[0][tid][1] = h16x4{0, 0, 0, 0};
    sm.Pb[3][tid][1] = h16x4{0, 0, 0, 0};
  }
  if constexpr (CV) {
    // This head's taps of q, k, v -> LDS (read by the helpers' tile loads).
    for (int i = tid; i < 3 * HD * 4; i += HNT) {
      const int sq = i / (HD * 4), e = i % (HD * 4);
      const float* src = sq == 0 ? ct.q : sq == 1 ? ct.k : ct.v;
      sm.tap[sq][(e & 3) * HD + (e >> 2)] = -kLog2e * src[(size_t)h * HD * 4 + e];
    }
    lds_barrier();
  }
  // Fragment rows 16 R .. 16 R + 15, 32-key step j: lane row lr, keys 32 j + 8 lq .. + 7.
  // The lane offsets are passed through an empty asm once per iteration
  // (lane_offset): otherwise the compiler hoists base + offset + constant out
  // of the loop as one register per read instead of folding the constants
  // into the instructions' offset fields.
  int fb = lr * HRS + 8 * lq;
  auto frag = [&](const h16* tile, int R, int j) { return ld8(tile + fb + 16 * R * HRS + 32 * j); };
  auto lane_offset = [](int& x) { asm volatile("" : "+v"(x)); };

  if (w < 4) {
    // ------------------------------------------------------- recurrence waves
    const int cw = w;
    // Transpose reads of K (token row 4 lq + lr / 4 + 16 r, keys 32 M + 8 (lr % 4) + 4 h)
    // and of av V (token rows 16 rt + 4 lq + lr / 4, columns of slice s).
    int tb = (4 * lq + (lr >> 2)) * HRS + 8 * (lr & 3);
    int vb = (4 * lq + (lr >> 2)) * HRS + 32 * cw + 4 * (lr & 3);
    f32x4 S[2][8];
    {
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[sl][m][i] = s0 ? s0[kap(m, 4 * lq + i) * HD + 32 * cw + 16 * sl + lr] : 0.f;
    }
    float sig = 1.f;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): state loads done before the loop
    for (int it = 0; it < NIT; ++it) {
      const int c2 = it - 2;
      const bool h2 = c2 >= 0 && c2 < NC;
      lane_offset(fb);
      lane_offset(tb);
      lane_offset(vb);
      // ---- phase 1: X~ = K S~, (Q S~)^T, Y~, U^ for both slices of chunk c2
      f32x4 X[2][4], QS[2][4];
      h16x4 u16[2][4];
      h16x8 udb[2][2];
      if (h2) {
        const h16* Kb = sm.K[c2 % 3];
        const HGate& gs = sm.g[c2 % 3];
        h16x8 sb[2][4];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
          for (int j = 0; j < 4; ++j) sb[sl][j] = cat8(cvt4(S[sl][2 * j]), cvt4(S[sl][2 * j + 1]));
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) X[sl][rt] = zero4(), QS[sl][rt] = zero4();
        // Per 32-key step: 4 K fragments (8 X products), 4 Q fragments (8
        // Q S products); the K fragments of step j + 1 are requested during
        // the X products of step j, the Q fragments during its Q S products.
        // Blocks (cw, 0) and (cw, 1) of P0 = lower(Q K^T) for the outputs of
        // phase 2, from the same K fragments and one more Q fragment per step
        // (wave 0's (0, 1) lies above the diagonal and is dropped); helpers 2
        // and 3 form (2, 2), (3, 2) and (3, 3).
        f32x4 GP[2] = {zero4(), zero4()};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h16x8 kf[4], qf[4];
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) kf[rt] = frag(Kb, rt, j);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) qf[rt] = frag(sm.Q, rt, j);
          const h16x8 qw = frag(sm.Q, cw, j);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) X[sl][rt] = mfma32(kf[rt], sb[sl][j], X[sl][rt]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) QS[sl][rt] = mfma32(sb[sl][j], qf[rt], QS[sl][rt]);
#pragma unroll
          for (int C = 0; C < 2; ++C) GP[C] = mfma32(kf[C], qw, GP[C]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 9, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 9, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 18, 0);
        {
          const bool widep = __builtin_amdgcn_readfirstlane(gs.wide) != 0;
          sm.Pb[pslot(cw, 0)][l][0] = p_block(gs, widep, cw, 0, GP[0], lr, lq, scale);
          if (cw >= 1) sm.Pb[pslot(cw, 1)][l][1] = p_block(gs, widep, cw, 1, GP[1], lr, lq, scale);
        }
        // Y~ = av V - (bx sigma) X~, U^ = T0 Y~ (av V and Tm of chunk c2 were
        // written in phase 2 of the previous iteration).
        const bool wide = __builtin_amdgcn_readfirstlane(gs.wide) != 0;
        const int s = c2 & 1;
        h16x4 va[2][4];
        f32x4 bv[4];
        h16x8 tc[6];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) va[sl][rt] = ld_tr(sm.V + vb + 16 * sl + 16 * rt * HRS);
          bv[rt] = ldf4(&gs.bx[16 * rt + 4 * lq]);
        }
#pragma unroll
        for (int i = 0; i < 6; ++i) tc[i] = sm.Tc[s][i][l];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          h16x4 y16[4];
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            f32x4 y;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = (float)va[sl][rt][i] - (bv[rt][i] * sig) * X[sl][rt][i];
            y16[rt] = cvt4(y);
          }
          const h16x8 ylo = cat8(y16[0], y16[1]), yhi = cat8(y16[2], y16[3]);
          f32x4 U[4];
          U[0] = mfma32(tc[0], ylo, zero4());
          U[1] = mfma32(tc[1], ylo, zero4());
          U[2] = mfma32(tc[2], ylo, zero4());
          U[3] = mfma32(tc[4], ylo, zero4());
          U[2] = mfma32(tc[3], yhi, U[2]);
          U[3] = mfma32(tc[5], yhi, U[3]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) u16[sl][rt] = cvt4(U[rt]);
          if (!wide) {
            udb[sl][0] = cat8(u16[sl][0], u16[sl][1]);
            udb[sl][1] = cat8(u16[sl][2], u16[sl][3]);
          } else {
            h16x4 d16[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) d16[rt] = cvt4(ldf4(&gs.dec[16 * rt + 4 * lq]) * U[rt]);
            udb[sl][0] = cat8(d16[0], d16[1]);
            udb[sl][1] = cat8(d16[2], d16[3]);
          }
        }
      }
      lds_barrier();
      // ---- phase 2: Y~, U^, S~ update, outputs of chunk c2
      f32x4 o[2][4];
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int R = 0; R < 4; ++R) o[sl][R] = zero4();
      if (h2) {
        const h16* Kb = sm.K[c2 % 3];
        const HGate& gs = sm.g[c2 % 3];
        const float rho = gs.gCc * sig;
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
          for (int m = 0; m < 8; ++m) S[sl][m] *= rho;
        // K^T fragments (keys 32 (m / 2) + 8 (lr % 4) + 4 (m % 2) .. + 3 of
        // token rows 4 lq + lr / 4 + 16 r) for the state update.
        h16x4 kt[8][4];
        auto ktr = [&](int m, int r) { return ld_tr(Kb + tb + 16 * r * HRS + 32 * (m >> 1) + 4 * (m & 1)); };
#pragma unroll
        for (int m = 0; m < 8; ++m) kt[m][0] = ktr(m, 0), kt[m][1] = ktr(m, 1);
        __builtin_amdgcn_sched_barrier(0);
        // S~ += K^T U^, breadth-first over the 16 state tiles; the second
        // half of the K^T fragments is read during the first half's products.
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const h16x8 k0 = cat8(kt[m][0], kt[m][1]);
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) S[sl][m] = mfma32(k0, udb[sl][0], S[sl][m]);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) kt[m][2] = ktr(m, 2), kt[m][3] = ktr(m, 3);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        h16x8 pb[6];
#pragma unroll
        for (int i = 0; i < 6; ++i) pb[i] = *reinterpret_cast<const h16x8*>(&sm.Pb[i][l][0]);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const h16x8 k1 = cat8(kt[m][2], kt[m][3]);
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) S[sl][m] = mfma32(k1, udb[sl][1], S[sl][m]);
        }
        // Outputs: (P U^)^T and (Q S~)^T hold token 16 R + lr, columns 4 lq + i.
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          const int t = 16 * R + lr;
          const float og = gs.og[t] * sig, of = gs.of[t];
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) {
            f32x4 PU = mfma32(cat8(u16[sl][0], u16[sl][1]), pb[pslot(R, 0)], zero4());
            if (R >= 2) PU = mfma32(cat8(u16[sl][2], u16[sl][3]), pb[pslot(R, 2)], PU);
#pragma unroll
            for (int i = 0; i < 4; ++i) o[sl][R][i] = og * QS[sl][R][i] + of * PU[i];
          }
        }
        sig = gs.cS;
      }
      {
        // Output rows of chunk c2 through a buffer resource covering its valid
        // rows only (stores past T or of a chunk out of range are dropped).
        const int nrows = h2 ? min(HC, Ts - c2 * HC) : 0;
        const TOut* cb = out + head0 + (size_t)max(c2, 0) * HC * tok;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<TOut*>(cb), (short)0, nrows * tok * (int)sizeof(TOut), 0x00020000);
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
          for (int R = 0; R < 4; ++R)
            store4<TOut>(rs, ((16 * R + lr) * tok + 32 * cw + 16 * sl + 4 * lq) * (int)sizeof(TOut),
                         o[sl][R]);
      }
      lds_barrier();
    }
    if (s_final) {
      float* dst = s_final;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dst[kap(m, 4 * lq + i) * HD + 32 * cw + 16 * sl + lr] = sig * S[sl][m][i];
    }
  } else {
    // ------------------------------------------------------------ helpers
    // The helpers carry the longer chain of dependent steps per phase; they
    // win instruction issue over the recurrence wave on their SIMD.
    __builtin_amdgcn_s_setprio(1);
    const int hw = w - 4, ht = tid - 256;
    const bf16* qh = q + head0;
    const bf16* kh = k + head0;
    const bf16* vh = v + head0;
    const float* ah = alpha + ((size_t)b * TS + (size_t)c0 * HC) * H + h;
    const float* bhp = beta + ((size_t)b * TS + (size_t)c0 * HC) * H + h;
    // Tile pieces of this thread: rows pr + 16 u (u = 0..3), 8 columns from pc.
    const int pr = ht >> 4, pc = (ht & 15) * 8;
    // Each iteration issues K 4 loads (phase 1), gates 2, Q 4, V 4 (phase
    // 2), in this order; a stream is consumed one iteration after its loads,
    // when 10 later operations (12 for the gates) have been issued.
    auto ld_tile = [&](const bf16* base, int c, bf16x8* r) {
      c = min(max(c, 0), NC - 1);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = min(c * HC + pr + 16 * u, Ts - 1);
        gld16(r[u], base + (size_t)t * tok + pc);
      }
    };
    const int st_off = pr * HRS + pc;
    auto st_tile = [&](h16* tile, const bf16x8* r) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<h16x8*>(tile + st_off + 16 * u * HRS) = bf16x8_to_h8(r[u]);
    };

    // Two register slots per stream (slot = iteration parity): a tile is
    // loaded two iterations before it goes to LDS.
    bf16x8 kr[2][4], qr[2][4], vr[2][4];
    float ra[2], rb[2];
    auto ld_gate = [&](int c, int p) {
      c = min(c, NC - 1);
      const int t = min(c * HC + l, Ts - 1);
      gld4(ra[p], ah + (size_t)t * H);
      gld4(rb[p], bhp + (size_t)t * H);
    };
    // Fused convolution: one register slot per stream, a tile's rows are
    // loaded one iteration before it goes to LDS.  Each iteration issues K 7
    // loads (phase 1), gates 2, Q 7, V 7 (phase 2), in this order; a stream
    // is consumed when 16 later operations (21 for the gates) have been
    // issued.
    ConvRows xk, xq, xv;
    const int cg = ht >> 4, tabs0 = c0 * HC;
    auto cissue = [&](ConvRows& x, const bf16* base, int c) {
      c = min(max(c, 0), NC - 1);
      conv_issue(x, base, c * HC, cg, pc, Ts, tabs0, tok);
    };
    auto cput = [&](const ConvRows& x, const float* taps, bool l2, int c, h16* tile,
                    const float* av) {
      float o[4][8], m[4];
      conv_rows(x, taps, pc, tabs0 + c * HC + 4 * cg - 3, tabs0 + c * HC < 3, l2, ct.eps, o, m);
      conv_store(tile, o, m, cg, pc, av);
    };
    if constexpr (CV) {
      cissue(xk, kh, 0);
      ld_gate(0, 0);
      cissue(xq, qh, -1);
      cissue(xv, vh, -1);
    } else {
      ld_tile(kh, 0, kr[0]);
      ld_tile(kh, 1, kr[1]);
      ld_gate(0, 0);
      ld_gate(1, 1);
      ld_tile(qh, 0, qr[1]);
      ld_tile(vh, 0, vr[1]);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // Each iteration issues K 4 loads (phase 1), gates 2, Q 4, V 4 (phase 2),
    // in this order; a stream is consumed two iterations after its loads,
    // when 24 later operations (26 for the gates) have been issued.
    auto wait24 = [&](bf16x8* r) {
      asm volatile("s_waitcnt vmcnt(24)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) :: "memory");
    };
    auto hbody = [&](int it, auto P) {
      constexpr int p = decltype(P)::value;  // it & 1
      const int c1 = it - 1, c2 = it - 2;
      const bool h1 = c1 >= 0 && c1 < NC;
      const bool h2 = c2 >= 0 && c2 < NC;
      lane_offset(fb);
      // ---- phase 1: K of chunk it -> LDS (slot it % 3 was last read in
      // phase 2 of it - 1)
      if constexpr (CV) {
        vm_wait_rows<16>(xk);
        if (it < NC) cput(xk, sm.tap[1], true, it, sm.K[it % 3], nullptr);
        cissue(xk, kh, it + 1);
      } else {
        wait24(kr[p]);
        if (it < NC) st_tile(sm.K[it % 3], kr[p]);
        ld_tile(kh, it + 2, kr[p]);
      }
      if (h1) {
        // Chunk c1: helper 0 forms the four diagonal blocks of A and inverts
        // them all (one lane per block column); helpers 1-3 form the
        // off-diagonal blocks, (1, 0), (2, 0), (2, 1) on helper 1, (3, 0),
        // (3, 1) on helper 2, (3, 2) on helper 3.
        const h16* Kb = sm.K[c1 % 3];
        const HGate& gs = sm.g[c1 % 3];
        const bool wide = __builtin_amdgcn_readfirstlane(gs.wide) != 0;
        if (hw == 0) {
          f32x4 G[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int R = 0; R < 4; ++R) {
              const h16x8 kf = frag(Kb, R, j);
              G[R] = mfma32(kf, kf, G[R]);
            }
#pragma unroll
          for (int R = 0; R < 4; ++R) {
            f32x4 Lb, LT;
            a_diag(gs, wide, R, G[R], lr, lq, Lb, LT);
            *reinterpret_cast<f32x4*>(sm.Iv4 + kInv4Block * R + kInv4Ld * lr + 4 * lq) = Lb;
          }
          inv16x4(sm.Iv4, l, &sm.Dg[0][0]);
        } else {
          f32x4 G0 = zero4(), G1 = zero4(), G2 = zero4();
          if (hw == 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const h16x8 k0 = frag(Kb, 0, j), k1 = frag(Kb, 1, j), k2 = frag(Kb, 2, j);
              G0 = mfma32(k0, k1, G0);  // (1, 0)
              G1 = mfma32(k0, k2, G1);  // (2, 0)
              G2 = mfma32(k1, k2, G2);  // (2, 1)
            }
            sm.Ab[0][l] = a_offdiag(gs, wide, 1, 0, G0, lr, lq);
            sm.Ab[1][l] = a_offdiag(gs, wide, 2, 0, G1, lr, lq);
            sm.Ab[2][l] = a_offdiag(gs, wide, 2, 1, G2, lr, lq);
          } else if (hw == 2) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const h16x8 k3 = frag(Kb, 3, j);
              G0 = mfma32(frag(Kb, 0, j), k3, G0);  // (3, 0)
              G1 = mfma32(frag(Kb, 1, j), k3, G1);  // (3, 1)
            }
            sm.Ab[3][l] = a_offdiag(gs, wide, 3, 0, G0, lr, lq);
            sm.Ab[4][l] = a_offdiag(gs, wide, 3, 1, G1, lr, lq);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) G0 = mfma32(frag(Kb, 2, j), frag(Kb, 3, j), G0);  // (3, 2)
            sm.Ab[5][l] = a_offdiag(gs, wide, 3, 2, G0, lr, lq);
          }
        }
      }
      if (hw >= 2 && h2) {
        // P blocks of chunk c2 on the block diagonal's lower right: (2, 2) on
        // helper 2, (3, 2) and (3, 3) on helper 3.
        const h16* Kb = sm.K[c2 % 3];
        const HGate& gs = sm.g[c2 % 3];
        const bool wide = __builtin_amdgcn_readfirstlane(gs.wide) != 0;
        f32x4 G0 = zero4(), G1 = zero4();
        if (hw == 2) {
#pragma unroll
          for (int j = 0; j < 4; ++j) G0 = mfma32(frag(Kb, 2, j), frag(sm.Q, 2, j), G0);
          sm.Pb[pslot(2, 2)][l][0] = p_block(gs, wide, 2, 2, G0, lr, lq, scale);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const h16x8 q3 = frag(sm.Q, 3, j);
            G0 = mfma32(frag(Kb, 2, j), q3, G0);
            G1 = mfma32(frag(Kb, 3, j), q3, G1);
          }
          sm.Pb[pslot(3, 2)][l][0] = p_block(gs, wide, 3, 2, G0, lr, lq, scale);
          sm.Pb[pslot(3, 3)][l][1] = p_block(gs, wide, 3, 3, G1, lr, lq, scale);
        }
      }
      lds_barrier();
      // ---- phase 2
      if (hw == 3 && h1) {
        h16x4 ga[6], d[7];
        h16x8 tc[6];
#pragma unroll
        for (int i = 0; i < 6; ++i) ga[i] = sm.Ab[i][l];
#pragma unroll
        for (int i = 0; i < 7; ++i) d[i] = sm.Dg[i][l];
        tm_offdiag(ga, d, tc);
#pragma unroll
        for (int i = 0; i < 6; ++i) sm.Tc[c1 & 1][i][l] = tc[i];
      }
      if constexpr (CV) {
        asm volatile("s_waitcnt vmcnt(21)" : "+v"(ra[0]), "+v"(rb[0]) :: "memory");
        if (hw == 2 && it < NC) gate_tables(sm.g[it % 3], ra[0], rb[0], it * HC + l < Ts, scale, l);
        ld_gate(it + 1, 0);
        vm_wait_rows<16>(xq);
        if (h1) cput(xq, sm.tap[0], true, c1, sm.Q, nullptr);
        cissue(xq, qh, it);
        vm_wait_rows<16>(xv);
        // av V of chunk c1 -> LDS (read by the recurrence waves in phase 1
        // of the next iteration).
        if (h1) cput(xv, sm.tap[2], false, c1, sm.V, sm.g[c1 % 3].av);
        cissue(xv, vh, it);
        lds_barrier();
        return;
      }
      asm volatile("s_waitcnt vmcnt(26)" : "+v"(ra[p]), "+v"(rb[p]) :: "memory");
      if (hw == 2 && it < NC) gate_tables(sm.g[it % 3], ra[p], rb[p], it * HC + l < Ts, scale, l);
      ld_gate(it + 2, p);
      wait24(qr[p]);
      if (h1) st_tile(sm.Q, qr[p]);
      ld_tile(qh, it + 1, qr[p]);
      wait24(vr[p]);
      if (h1) {
        // av V of chunk c1 -> LDS (read by the recurrence waves in phase 1 of
        // the next iteration).
        const HGate& gs = sm.g[c1 % 3];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float a = gs.av[pr + 16 * u];
          h16x8 x;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (h16)(a * (float)vr[p][u][e]);
          *reinterpret_cast<h16x8*>(sm.V + st_off + 16 * u * HRS) = x;
        }
      }
      ld_tile(vh, it + 1, vr[p]);
      lds_barrier();
    };
    // Odd last iteration peeled, as in the transition pass.
    int it = 0;
    for (; it + 1 < NIT; it += 2) {
      hbody(it, ic<0>());
      hbody(it + 1, ic<1>());
    }
    if (it < NIT) hbody(it, ic<0>());
    if constexpr (CV) {
      vm_wait_rows<0>(xk);
      vm_wait_rows<0>(xq);
      vm_wait_rows<0>(xv);
    } else {
      vm_drain(kr);
      vm_drain(qr);
      vm_drain(vr);
    }
    vm_drain(ra, rb);
  }
}

union __align__(16) PrefillSmem {
  TSmem t;
  HSmem h;
};

// Segments 0 .. P - 2 of a segmented prefill (work-group = head * (P - 1) +
// s): s = 0 runs the output pass of segment 0 from the state in and leaves
// its final state, the initial state of segment 1, in the workspace; s >= 1
// runs the transition pass of segment s.
template <class TOut, bool CV>
__global__ __launch_bounds__(HNT) void prefill_lead_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* state_in,
    TOut* __restrict__ out, SegWs ws, SegGeom g, int T, int TS, int H, float scale,
    ConvTaps ct) {
  __shared__ PrefillSmem sm;
  const int bh = blockIdx.x / (g.P - 1), s = blockIdx.x % (g.P - 1);
  const int b = bh / H, h = bh % H;
  if (s == 0) {
    out_segment<TOut, CV>(sm.h, q, k, v, alpha, beta,
                          state_in ? state_in + (size_t)bh * HD * HD : nullptr,
                          ws.S + ws.at(bh, 0, g.P), out, b, h, T, TS, H, 0, g.count(0), scale, ct);
  } else {
    transition_segment<CV>(sm.t, k, v, alpha, beta, ws.B + ws.at(bh, s, g.P),
                           ws.M + ws.at(bh, s, g.P), b, h, T, TS, H, g.first(s), g.count(s), ct);
  }
}

// Output pass of segments s_first .. P - 1 (work-group = head * (P - s_first)
// + s - s_first) from their initial states (segment 0: the state in; others:
// the workspace); segment P - 1 writes the final state.
template <class TOut, bool CV>
__global__ __launch_bounds__(HNT) void prefill_out_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* state_in,
    float* state_out, TOut* __restrict__ out, SegWs ws, SegGeom g, int s_first, int T, int TS,
    int H, float scale, ConvTaps ct) {
  __shared__ HSmem sm;
  const int n = g.P - s_first;
  const int bh = blockIdx.x / n, s = s_first + blockIdx.x % n;
  const int b = bh / H, h = bh % H;
  const float* s0 = s == 0 ? (state_in ? state_in + (size_t)bh * HD * HD : nullptr)
                           : ws.S + ws.at(bh, s - 1, g.P);
  float* sf = (s == g.P - 1 && state_out) ? state_out + (size_t)bh * HD * HD : nullptr;
  out_segment<TOut, CV>(sm, q, k, v, alpha, beta, s0, sf, out, b, h, T, TS, H, g.first(s),
                        g.count(s), scale, ct);
}

// Initial states of segments 2 .. P - 1: from S_1 (left in the workspace by
// the output pass of segment 0), S_{s+1} = M_s S_s + B_s, in f32.  One
// work-group per (head, 16-column slice); wave w forms RT row tiles (16 rows
// each, tiles RT w .. RT w + RT - 1) of every step with
// v_mfma_f32_16x16x4_f32: in the 16-key block jj, product i takes key 16 jj
// + 4 q + i in lane group q, so each lane reads its 4 keys of M with one
// 16-byte load and S (kept transposed in LDS) with one 16-byte read; each
// row tile accumulates in two chains (even and odd key blocks).
//   - PF (the grid fits two work-groups per CU): 8 waves, one row tile each;
//     the next segment's M and B are requested (inline asm, 12 loads per
//     lane, two register slots) before the current product, and each step's
//     result is written with 4 vector stores (inline asm): at the end of a
//     step the loads are complete once at most those 4 stores are
//     outstanding, so no wait covers a store.
//   - otherwise: 4 waves, two row tiles each, one register slot (under 128
//     VGPRs, so four work-groups fit per CU and the grid runs in one round);
//     each step waits for its own loads.
__device__ __forceinline__ void cb_ld4(f32x4& r, const float* p) {
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
}
__device__ __forceinline__ void cb_ld1(float& r, const float* p) {
  asm volatile("global_load_dword %0, %1, off" : "=v"(r) : "v"(p) : "memory");
}
__device__ __forceinline__ void cb_st1(float* p, float v) {
  asm volatile("global_store_dword %0, %1, off" : : "v"(p), "v"(v) : "memory");
}
template <int RT>
struct CombLoads {
  f32x4 m[RT][8];  // M rows 16 (RT w + t) + lr, keys 16 jj + 4 lq .. + 3
  float b[RT][4];  // B in accumulator layout: rows 16 (RT w + t) + 4 lq + i, column lr
};
template <int N>
__device__ __forceinline__ void cb_wait(CombLoads<1>& x) {
  asm volatile("s_waitcnt vmcnt(%12)"
               : "+v"(x.m[0][0]), "+v"(x.m[0][1]), "+v"(x.m[0][2]), "+v"(x.m[0][3]),
                 "+v"(x.m[0][4]), "+v"(x.m[0][5]), "+v"(x.m[0][6]), "+v"(x.m[0][7]),
                 "+v"(x.b[0][0]), "+v"(x.b[0][1]), "+v"(x.b[0][2]), "+v"(x.b[0][3])
               : "n"(N)
               : "memory");
}
template <int N>
__device__ __forceinline__ void cb_wait(CombLoads<2>& x) {
  asm volatile("s_waitcnt vmcnt(%24)"
               : "+v"(x.m[0][0]), "+v"(x.m[0][1]), "+v"(x.m[0][2]), "+v"(x.m[0][3]),
                 "+v"(x.m[0][4]), "+v"(x.m[0][5]), "+v"(x.m[0][6]), "+v"(x.m[0][7]),
                 "+v"(x.m[1][0]), "+v"(x.m[1][1]), "+v"(x.m[1][2]), "+v"(x.m[1][3]),
                 "+v"(x.m[1][4]), "+v"(x.m[1][5]), "+v"(x.m[1][6]), "+v"(x.m[1][7]),
                 "+v"(x.b[0][0]), "+v"(x.b[0][1]), "+v"(x.b[0][2]), "+v"(x.b[0][3]),
                 "+v"(x.b[1][0]), "+v"(x.b[1][1]), "+v"(x.b[1][2]), "+v"(x.b[1][3])
               : "n"(N)
               : "memory");
}

template <bool PF>
__global__ __launch_bounds__(PF ? 512 : 256) void segment_combine_kernel(SegWs ws, int P) {
  constexpr int RT = PF ? 1 : 2;   // row tiles per wave
  constexpr int NT = 64 * 8 / RT;  // threads
  __shared__ __align__(16) float St[16][HD + 4];  // S slice transposed: [column][key]
  // The 8 slices of a head on one XCD (when the head count is a multiple of
  // 8), so M_s comes from HBM into one L2 once and is read from there 8 times.
  int bh, sl;
  xcd_group_map(blockIdx.x, gridDim.x / 8, 8, &bh, &sl);
  const int col0 = 16 * sl;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lq = l >> 4;
  const float* s1 = ws.S + ws.at(bh, 0, P);
  for (int i = tid; i < HD * 16; i += NT) {
    const int r = i >> 4, c = i & 15;
    St[c][r] = s1[r * HD + col0 + c];
  }
  const int last = P - 2;  // steps sg = 1 .. last
  auto issue = [&](CombLoads<RT>& x, int sg) {
    sg = min(sg, last);
    const float* M = ws.M + ws.at(bh, sg, P);
    const float* Bs = ws.B + ws.at(bh, sg, P);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int row = 16 * (RT * w + t) + lr;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) cb_ld4(x.m[t][jj], M + (size_t)row * HD + 16 * jj + 4 * lq);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        cb_ld1(x.b[t][i], Bs + (size_t)(16 * (RT * w + t) + 4 * lq + i) * HD + col0 + lr);
    }
  };
  CombLoads<RT> ld[PF ? 2 : 1];
  issue(ld[0], 1);
  cb_wait<0>(ld[0]);  // also covers the compiler's loads of S_1 above
  lds_barrier();
  auto step = [&](int sg, auto Par) {
    constexpr int p = decltype(Par)::value;  // (sg - 1) & 1
    if constexpr (PF) issue(ld[p ^ 1], sg + 1);
    f32x4 acc[RT][2];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      acc[t][0] = f32x4{ld[p].b[t][0], ld[p].b[t][1], ld[p].b[t][2], ld[p].b[t][3]};
      acc[t][1] = zero4();
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const f32x4 sv = ldf4(&St[lr][16 * jj + 4 * lq]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[t][jj & 1] =
              __builtin_amdgcn_mfma_f32_16x16x4f32(ld[p].m[t][jj][i], sv[i], acc[t][jj & 1], 0, 0, 0);
      }
    }
    lds_barrier();  // every wave has read St
    float* dst = ws.S + ws.at(bh, sg, P);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const f32x4 a = acc[t][0] + acc[t][1];
      const int r0 = 16 * (RT * w + t) + 4 * lq;
      *reinterpret_cast<f32x4*>(&St[lr][r0]) = a;
#pragma unroll
      for (int i = 0; i < 4; ++i) cb_st1(dst + (size_t)(r0 + i) * HD + col0 + lr, a[i]);
    }
    lds_barrier();
    if constexpr (PF) cb_wait<4 * RT>(ld[p ^ 1]);
  };
  if constexpr (PF) {
    int sg = 1;
    for (; sg + 1 <= last; sg += 2) {
      step(sg, ic<0>());
      step(sg + 1, ic<1>());
    }
    if (sg <= last) step(sg, ic<0>());
  } else {
    for (int sg = 1; sg <= last; ++sg) {
      if (sg > 1) {
        issue(ld[0], sg);
        cb_wait<0>(ld[0]);
      }
      step(sg, ic<0>());
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last stores
  cb_wait<0>(ld[0]);
  if constexpr (PF) cb_wait<0>(ld[1]);
}

}  // namespace

bool prefill_head_supported(const PrefillArgs& p) {
  return p.bf16 && p.Dk == HD && p.Dv == HD && p.chunk == HC && p.T > 0;
}
// The fused convolution additionally reads each sequence's rows from its
// start (no history before token 0), so sequences must be dense.
bool prefill_head_conv_supported(const PrefillArgs& p) {
  return prefill_head_supported(p) && (p.seq_stride == 0 || p.seq_stride == p.T);
}

// Segments per head.  Both segmented launches (the output pass of segment 0
// beside the transition passes of segments 1 .. P - 2, then the output passes
// of segments 1 .. P - 1) have B H (P - 1) work-groups, at most one per CU
// (the kernels hold 120-143 KB of LDS).  Segment 0 gets kLeadRatio times the
// chunks of the others -- about the transition pass's cost per chunk
// relative to the output pass's -- so both kinds of work-group in the first
// launch finish together.  Segments average at least kMinSegChunks chunks;
// fewer than 3 segments do not shorten the serial chain.
constexpr int kCUs = 256;
constexpr int kMinSegChunks = 8;
constexpr double kLeadRatio = 0.9;
void prefill_head_segments(int B, int T, int H, int* P, int* L0, int* L) {
  const int NC = (T + HC - 1) / HC;
  const long long BH = std::max(1LL, (long long)B * H);
  int p = (int)std::min<long long>(1 + kCUs / BH, NC / kMinSegChunks);
  if (p < 3) {
    *P = 1;
    *L0 = *L = NC;
    return;
  }
  const int l = (int)std::ceil(NC / (p - 1 + kLeadRatio));
  int l0 = NC - (p - 1) * l;
  if (l0 < 1) {  // rounding left segment 0 empty: give it its share, drop the surplus
    l0 = std::max(1, (int)(kLeadRatio * l));
    p = 1 + (NC - l0 + l - 1) / l;
  }
  *P = p;
  *L0 = l0;
  *L = l;
}

size_t prefill_head_workspace_bytes(int B, int T, int H) {
  int P, L0, L;
  prefill_head_segments(B, T, H, &P, &L0, &L);
  if (P <= 1) return 0;
  return 3 * (size_t)B * H * (P - 1) * HD * HD * sizeof(float);
}

template <class TOut, bool CV>
static hipError_t launch_head_t(const PrefillArgs& p) {
  const ConvTaps ct{p.taps_q, p.taps_k, p.taps_v, p.conv_eps};
  SegGeom g;
  g.NCT = (p.T + HC - 1) / HC;
  prefill_head_segments(p.B, p.T, p.H, &g.P, &g.L0, &g.L);
  const int BH = p.B * p.H;
  const int TS = p.seq_stride > 0 ? p.seq_stride : p.T;  // tokens between sequence starts
  SegWs ws{nullptr, nullptr, nullptr};
  const hipStream_t st = (hipStream_t)p.stream;
  const bf16 *q = (const bf16*)p.q, *k = (const bf16*)p.k, *v = (const bf16*)p.v;
  int s_first = 0;
  if (g.P > 1) {
    const size_t n = (size_t)BH * (g.P - 1) * HD * HD;
    ws.M = (float*)p.workspace;
    ws.B = ws.M + n;
    ws.S = ws.B + n;
    hipLaunchKernelGGL((prefill_lead_kernel<TOut, CV>), dim3(BH * (g.P - 1)), dim3(HNT), 0, st, q,
                       k, v, p.alpha, p.beta, p.state_in, (TOut*)p.out, ws, g, p.T, TS, p.H,
                       p.scale, ct);
    if (g.P > 2) {
      if (BH * 8 <= 2 * kCUs)
        hipLaunchKernelGGL(segment_combine_kernel<true>, dim3(BH * 8), dim3(512), 0, st, ws, g.P);
      else
        hipLaunchKernelGGL(segment_combine_kernel<false>, dim3(BH * 8), dim3(256), 0, st, ws, g.P);
    }
    s_first = 1;
  }
  hipLaunchKernelGGL((prefill_out_kernel<TOut, CV>), dim3(BH * (g.P - s_first)), dim3(HNT), 0, st,
                     q, k, v, p.alpha, p.beta, p.state_in, p.state_out, (TOut*)p.out, ws, g,
                     s_first, p.T, TS, p.H, p.scale, ct);
  return hipGetLastError();
}

hipError_t launch_prefill_head(const PrefillArgs& p) {
  if (p.taps_q) return p.out_bf16 ? launch_head_t<bf16, true>(p) : launch_head_t<float, true>(p);
  return p.out_bf16 ? launch_head_t<bf16, false>(p) : launch_head_t<float, false>(p);
}

}  // namespace gdn
