// f16 MFMA building blocks of the chunked prefill kernels (gfx950).
//
// Operand layouts.  A 16x16 MFMA result is held by lane l = 16 q + r as rows
// 4 q .. 4 q + 3 of column r (accumulator layout, written D(M)).  The
// A-operand fragment of M is D(M^T), the B-operand fragment is D(M), so
// D(M N) = mfma(D(M^T), D(N)) and D((M N)^T) = mfma(D(N), D(M^T)).  A 32-deep
// product (v_mfma_f32_16x16x32_f16) takes 8 contraction values per lane; which
// logical index sits in which lane slot is free as long as both operands
// agree, so two stacked accumulator tiles can serve as one operand.
#pragma once

#include <type_traits>

#include "gdn_device.h"

namespace gdn {
namespace f16ops {

typedef _Float16 h16;
typedef h16 h16x4 __attribute__((ext_vector_type(4)));
typedef h16 h16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
template <int V>
using ic = std::integral_constant<int, V>;

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
// bf16 -> f16 of four values.  Every bf16 value in the f16 normal range is
// exactly representable, so the packed round-toward-zero conversion is exact
// there (and only flushes magnitudes below 2^-14 towards zero).
__device__ __forceinline__ h16x4 bf16_to_h4(bf16x4 x) {
  typedef h16 h16x2 __attribute__((ext_vector_type(2)));
  const h16x2 a = __builtin_bit_cast(h16x2, __builtin_amdgcn_cvt_pkrtz((float)x[0], (float)x[1]));
  const h16x2 b = __builtin_bit_cast(h16x2, __builtin_amdgcn_cvt_pkrtz((float)x[2], (float)x[3]));
  return h16x4{a[0], a[1], b[0], b[1]};
}
__device__ __forceinline__ h16x8 cvt8(bf16x4 lo, bf16x4 hi) {
  return cat8(bf16_to_h4(lo), bf16_to_h4(hi));
}
__device__ __forceinline__ h16x8 bf16x8_to_h8(bf16x8 x) {
  return cvt8(__builtin_shufflevector(x, x, 0, 1, 2, 3), __builtin_shufflevector(x, x, 4, 5, 6, 7));
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
// Work-group barrier ordering LDS only.  Waves exchange data through LDS
// alone, so global loads issued for later chunks stay in flight across it
// (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (lanes read as zero where the shifted source is absent).
__device__ __forceinline__ float wave_incl_sum(float x) {
  const int z = 0;
  auto sh = [&](float v, auto ctrl) -> float {
    constexpr int C = decltype(ctrl)::value;
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(z, __builtin_bit_cast(int, v), C, 0xf, 0xf, false));
  };
  x += sh(x, ic<0x111>());  // row_shr:1
  x += sh(x, ic<0x112>());  // row_shr:2
  x += sh(x, ic<0x114>());  // row_shr:4
  x += sh(x, ic<0x118>());  // row_shr:8
  // row_bcast:15 adds lane 15 of each row to the next row; row_bcast:31 adds
  // lane 31 to rows 2 and 3.
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(z, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(z, __builtin_bit_cast(int, x), 0x143, 0xc, 0xf, false));
  return x;
}
// Lane group p's value (16 lanes) broadcast to every lane group, same lane
// within the group.  v_permlane16_swap exchanges odd rows of its first
// operand with even rows of its second (with both = x: {x0, x0, x2, x2} and
// {x1, x1, x3, x3}); v_permlane32_swap exchanges the upper half of the first
// with the lower half of the second (with both = s: {s0, s1, s0, s1} and
// {s2, s3, s2, s3}).
template <int P>
__device__ __forceinline__ float bcast_group(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned s = (P & 1) ? a[1] : a[0];
  const auto b = __builtin_amdgcn_permlane32_swap(s, s, false, false);
  return __builtin_bit_cast(float, (P & 2) ? b[1] : b[0]);
}

// LDS scratch of inv16 per wave (floats): L row-major and the solution
// column-major, 16 x 16 f32 each with a row stride of 20 floats (the reads
// then touch distinct banks).
constexpr int kInvLd = 20;
constexpr int kInvScratch = 2 * 16 * kInvLd;

// T = (I + L)^-1 for a strictly lower 16x16 L, by forward substitution in
// f32.  The product form (I + L^8)(I + L^4)(I + L^2)(I - L) is not used: when
// keys cluster around one direction the powers of L grow to hundreds or
// thousands and cancel, and their rounding swamps T.  In: D(L^T) (the
// accumulator layout of L^T).  Out: D(T), D(T^T) (f32).  scr: this wave's LDS
// scratch, kInvScratch floats, 16-byte aligned, used by no other wave.
// Lane (lq, lr) solves rows 4 lq .. 4 lq + 3 of column lr of (I + L) T = I,
// in four steps over row blocks p = 0..3: block p is final once it has
// taken its 4 x 4 diagonal solve; it is broadcast across the lane groups
// (cross-lane swaps), and every later block subtracts L[its rows][4 p ..
// 4 p + 3] times it.  T then goes through the scratch column-major, from
// which D(T^T) is read.
__device__ __forceinline__ void inv16(f32x4 LTf, int lr, int lq, float* scr, f32x4& T, f32x4& TT) {
  float* Lm = scr;                // Lm[r][i] = L[r][i]
  float* Xc = scr + 16 * kInvLd;  // Xc[c][r] = T[r][c]
  // Lane (lq, lr) holds L^T[4 lq + j][lr] = L[lr][4 lq + j], j = 0..3.
  *reinterpret_cast<f32x4*>(Lm + kInvLd * lr + 4 * lq) = LTf;
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = (4 * lq + j == lr) ? 1.f : 0.f;
  // L[4 lq + j][4 p .. 4 p + 3] for j = 0..3.
  auto lblk = [&](int p, f32x4* m) {
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = *reinterpret_cast<const f32x4*>(Lm + kInvLd * (4 * lq + j) + 4 * p);
  };
  f32x4 m[4][4];
#pragma unroll
  for (int p = 0; p < 4; ++p) lblk(p, m[p]);
  auto step = [&](auto P) {
    constexpr int p = decltype(P)::value;
    if (lq == p) {
      // 4 x 4 diagonal block: x_j -= sum_{i < j} L[4 p + j][4 p + i] x_i.
#pragma unroll
      for (int j = 1; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < j; ++i) x[j] = __builtin_fmaf(-m[p][j][i], x[i], x[j]);
    }
    if constexpr (p < 3) {
      // Rows of later blocks: x_j -= sum_i L[4 lq + j][4 p + i] T[4 p + i][lr].
      f32x4 xp;
#pragma unroll
      for (int i = 0; i < 4; ++i) xp[i] = bcast_group<p>(x[i]);
      if (lq > p) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[j] = __builtin_fmaf(-m[p][j][i], xp[i], x[j]);
      }
    }
  };
  step(ic<0>());
  step(ic<1>());
  step(ic<2>());
  step(ic<3>());
  T = x;  // T[4 lq + j][lr]
  *reinterpret_cast<f32x4*>(Xc + kInvLd * lr + 4 * lq) = x;
#pragma unroll
  for (int j = 0; j < 4; ++j) TT[j] = Xc[kInvLd * (4 * lq + j) + lr];  // T[lr][4 lq + j]
}

// The four diagonal 16 x 16 blocks of a 64-token chunk's Tm = (I + A)^-1, on
// one wave, by forward substitution in f32: lane 16 b + c solves
// (I + L_b) x = e_c for column c of block b (column axpy form: once x_i is
// final, x_r -= L_b[r][i] x_i for r > i).  The strictly lower blocks L_b
// arrive column-major in the wave's LDS scratch: lcm + kInv4Block b + 20 i
// holds L_b[0..15][i] (the caller writes D(L_b) there, one 16-byte store per
// lane and block).  Out: the f16 operands dg = {D(T00), D(T00^T), D(T11),
// D(T11^T), D(T22), D(T22^T), D(T33^T)} (h16x4 per lane, 64 lanes each).
constexpr int kInv4Ld = 20;                   // floats per column
constexpr int kInv4Block = 16 * kInv4Ld + 4;  // floats per block (bank offset 4)
constexpr int kInv4Scratch = 4 * kInv4Block;
__device__ __forceinline__ void inv16x4(const float* lcm, int l, h16x4* dg) {
  const int b = l >> 4, c = l & 15;
  const float* P = lcm + kInv4Block * b;
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
  auto col = [&](int i, f32x4* v) {
#pragma unroll
    for (int q = (i + 1) >> 2; q < 4; ++q) v[q] = *reinterpret_cast<const f32x4*>(P + kInv4Ld * i + 4 * q);
  };
  // Columns are read two steps ahead of their use (three in flight).
  f32x4 buf[3][4];
  col(0, buf[0]);
  col(1, buf[1]);
#pragma unroll
  for (int i = 0; i < 15; ++i) {
    if (i + 2 < 15) col(i + 2, buf[(i + 2) % 3]);
#pragma unroll
    for (int r = i + 1; r < 16; ++r) x[r] = __builtin_fmaf(-buf[i % 3][r >> 2][r & 3], x[i], x[r]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // D(T_b): lane (q, c) of the operand holds T_b[4 q .. 4 q + 3][c], i.e.
  // x[4 q .. 4 q + 3] of this lane.  D(T_b^T): lane (q, c') holds
  // T_b[c'][4 q + j] = x[c'] of lane (b, 4 q + j).
  const int nb = b < 3 ? 2 * b : -1;       // D(T_b) slot (none for b = 3)
  const int tb = b < 3 ? 2 * b + 1 : 6;    // D(T_b^T) slot
  if (nb >= 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dg[64 * nb + 16 * q + c] = h16x4{(h16)x[4 * q], (h16)x[4 * q + 1], (h16)x[4 * q + 2], (h16)x[4 * q + 3]};
  }
  h16* dt = reinterpret_cast<h16*>(dg + 64 * tb);
#pragma unroll
  for (int r = 0; r < 16; ++r) dt[4 * (16 * (c >> 2) + r) + (c & 3)] = (h16)x[r];
}

// Off-diagonal blocks of the unit lower triangular Tm = (I + A)^-1 of a
// 64-token chunk by block forward substitution, from the A-operand fragments
// of the strictly lower blocks of A and the diagonal inverses:
//   T10 = -T11 A10 T00,  T32 = -T33 A32 T22,
//   T2j = -T22 Z2j,  T3j = -(T32 Z2j + T33 Z3j),  Zmj = Am0 T0j + Am1 T1j.
// ga = {A10, A20, A21, A30, A31, A32}; d = {D(T00), D(T00^T), D(T11),
// D(T11^T), D(T22), D(T22^T), D(T33^T)}.  Out: the six A operands of Tm for
// the 64 x 16 product Tm Y with Y as two 32-row operands (row tile, step):
//   tc[0] = (0,0) [T00 | 0]    tc[1] = (1,0) [T10 | T11]
//   tc[2] = (2,0) [T20 | T21]  tc[3] = (2,1) [T22 | 0]
//   tc[4] = (3,0) [T30 | T31]  tc[5] = (3,1) [T32 | T33]
__device__ __forceinline__ void tm_offdiag(const h16x4 ga[6], const h16x4 d[7], h16x8 tc[6]) {
  const h16x4 d00 = d[0], d00t = d[1], d11 = d[2], d11t = d[3];
  const h16x4 d22 = d[4], d22t = d[5], d33t = d[6];
  const h16x4 x10 = cvt4(mfma16(ga[0], d00, zero4()));   // D(A10 T00)
  const h16x4 t10t = cvt4(-mfma16(x10, d11t, zero4()));  // D(T10^T)
  const h16x4 t10 = cvt4(-mfma16(d11t, x10, zero4()));   // D(T10)
  const h16x4 x32 = cvt4(mfma16(ga[5], d22, zero4()));   // D(A32 T22)
  const h16x4 t32t = cvt4(-mfma16(x32, d33t, zero4()));  // D(T32^T)
  const h16x8 d0010 = cat8(d00, t10);
  const h16x4 z20 = cvt4(mfma32(cat8(ga[1], ga[2]), d0010, zero4()));
  const h16x4 z30 = cvt4(mfma32(cat8(ga[3], ga[4]), d0010, zero4()));
  const h16x4 z21 = cvt4(mfma16(ga[2], d11, zero4()));
  const h16x4 z31 = cvt4(mfma16(ga[4], d11, zero4()));
  const h16x4 t20t = cvt4(-mfma16(z20, d22t, zero4()));
  const h16x4 t21t = cvt4(-mfma16(z21, d22t, zero4()));
  const h16x8 t3233 = cat8(t32t, d33t);
  const h16x4 t30t = cvt4(-mfma32(cat8(z20, z30), t3233, zero4()));
  const h16x4 t31t = cvt4(-mfma32(cat8(z21, z31), t3233, zero4()));
  const h16x4 zz = {0, 0, 0, 0};
  tc[0] = cat8(d00t, zz);
  tc[1] = cat8(t10t, d11t);
  tc[2] = cat8(t20t, t21t);
  tc[3] = cat8(d22t, zz);
  tc[4] = cat8(t30t, t31t);
  tc[5] = t3233;
}

}  // namespace f16ops
}  // namespace gdn
