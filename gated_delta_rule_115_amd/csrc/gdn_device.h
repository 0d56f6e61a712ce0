// Device-side building blocks shared by the gfx950 kernels of the GDN library.
//
// Matrix products use the CDNA4 16x16-output MFMA family:
//   bf16: v_mfma_f32_16x16x32_bf16  (each lane holds 8 consecutive k values)
//   f16:  v_mfma_f32_16x16x32_f16   (same shape, 3 more mantissa bits)
//   f32:  v_mfma_f32_16x16x4_f32    (each lane holds 1 k value)
// Operand layout (both A and B are read "k-contiguous", i.e. A as [m][k] and
// B as [n][k]):  lane l supplies row/column (l % 16) and k values
// k0 + (l / 16) * KPL + (0 .. KPL-1).  The 16x16 f32 result tile is held as
// 4 floats per lane: lane l holds rows 4*(l/16) + i, i = 0..3, of column l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

template <class T>
struct Mfma;

template <>
struct Mfma<bf16> {
  static constexpr int KSTEP = 32;  // contraction depth of one instruction
  static constexpr int KPL = 8;     // contraction values per lane
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag zero() {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (bf16)0.0f;
    return f;
  }
};

template <>
struct Mfma<f16> {
  static constexpr int KSTEP = 32;
  static constexpr int KPL = 8;
  typedef f16x8 frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag zero() {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (f16)0.0f;
    return f;
  }
};

// Operand type of the state-path products for a given input type: bf16
// inputs use f16 operands (exact for unit-scale bf16 values, 8x finer
// rounding of the intermediate S, Y, U, Tm, Pm); f32 inputs stay f32.
template <class TIn>
struct OperandOf {
  typedef f16 type;
};
template <>
struct OperandOf<float> {
  typedef float type;
};

template <>
struct Mfma<float> {
  static constexpr int KSTEP = 4;
  static constexpr int KPL = 1;
  typedef float frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag zero() { return 0.0f; }
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Operand fragment from a k-contiguous array: element (r, kk) at
// base[r * ld + kk], r = l % 16.  Lanes whose k range starts at or beyond
// `klimit` get zeros (zero padding of a short contraction; klimit % KPL == 0).
template <class T>
__device__ __forceinline__ typename Mfma<T>::frag frag_k(const T* base, int ld,
                                                         int k0, int klimit) {
  const int l = lane_id();
  const int kk = k0 + (l >> 4) * Mfma<T>::KPL;
  if (kk >= klimit) return Mfma<T>::zero();
  return *reinterpret_cast<const typename Mfma<T>::frag*>(base + (l & 15) * ld + kk);
}

// Operand fragment from an m-contiguous array (the transpose of frag_k):
// element (r, kk) at base[kk * ld + r].  Used where the contraction runs over
// the slow index of the stored tile.
template <class T>
__device__ __forceinline__ typename Mfma<T>::frag frag_m(const T* base, int ld,
                                                         int k0, int klimit) {
  const int l = lane_id();
  const int kk = k0 + (l >> 4) * Mfma<T>::KPL;
  typename Mfma<T>::frag f = Mfma<T>::zero();
  if (kk >= klimit) return f;
  const T* p = base + kk * ld + (l & 15);
  if constexpr (Mfma<T>::KPL == 1) {
    f = p[0];
  } else {
#pragma unroll
    for (int i = 0; i < Mfma<T>::KPL; ++i) f[i] = p[i * ld];
  }
  return f;
}

template <class T>
__device__ __forceinline__ T from_f32(float x) {
  return static_cast<T>(x);
}

template <class T>
__device__ __forceinline__ float to_f32(T x) {
  return static_cast<float>(x);
}

// 16-byte vector of T (8 bf16 or 4 f32).
template <class T>
struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
  typedef T type __attribute__((ext_vector_type(N)));
};

// Raw per-lane operand bits as loaded from memory (KPL elements of the input
// type), converted to an MFMA fragment of the operand type only when used.
template <class TIn, int KPL>
struct RawFrag {
  typedef TIn type __attribute__((ext_vector_type(KPL)));
  static __device__ __forceinline__ type zero() {
    type r;
#pragma unroll
    for (int e = 0; e < KPL; ++e) r[e] = static_cast<TIn>(0.0f);
    return r;
  }
  template <class OpT>
  static __device__ __forceinline__ typename Mfma<OpT>::frag to_frag(type r) {
    typename Mfma<OpT>::frag f;
#pragma unroll
    for (int e = 0; e < KPL; ++e) f[e] = static_cast<OpT>(static_cast<float>(r[e]));
    return f;
  }
};
template <class TIn>
struct RawFrag<TIn, 1> {
  typedef TIn type;
  static __device__ __forceinline__ type zero() { return static_cast<TIn>(0.0f); }
  template <class OpT>
  static __device__ __forceinline__ typename Mfma<OpT>::frag to_frag(type r) {
    return static_cast<OpT>(static_cast<float>(r));
  }
};

// One element loaded into its own 32-bit register without conversion (bf16:
// zero-extended bits; f32: the bits), so the load can stay in flight until
// raw32_to_f32 is applied.
template <class T>
__device__ __forceinline__ uint32_t load_raw32(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return (uint32_t)(*reinterpret_cast<const unsigned short*>(p));
  } else {
    return *reinterpret_cast<const uint32_t*>(p);
  }
}
template <class T>
__device__ __forceinline__ float raw32_to_f32(uint32_t r) {
  if constexpr (sizeof(T) == 2) {
    return __uint_as_float(r << 16);  // bf16 -> f32 is exact
  } else {
    return __uint_as_float(r);
  }
}

// Map a block index to (group, member) so that the `members` blocks of one
// group land on the same XCD.  Work-groups are dispatched round-robin over the
// 8 XCDs (block i -> XCD i % 8); keeping one head's blocks on one XCD lets
// them share that XCD's L2 copy of the head's inputs.  Falls back to a plain
// split when the group count is not a multiple of 8.
__device__ __forceinline__ void xcd_group_map(int bid, int groups, int members,
                                              int* group, int* member) {
  if ((groups & 7) == 0 && members > 1) {
    const int xcd = bid & 7;
    const int j = bid >> 3;
    *group = (j / members) * 8 + xcd;
    *member = j % members;
  } else {
    *group = bid / members;
    *member = bid % members;
  }
}

}  // namespace gdn
