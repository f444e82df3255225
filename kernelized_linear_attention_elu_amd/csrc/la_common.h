// Device-side building blocks shared by the linear-attention kernels (gfx950).
//
// Conventions
//  * A workgroup is 256 threads = 4 wave64s.  In a wave, lane l is split into
//    g = l / 16 (0..3) and li = l % 16.
//  * 16x16 MFMA tiles.  For D = A(16xK) * B(Kx16) + C the operand lanes are:
//      A: lane (g, li) supplies row li, k-slots owned by group g;
//      B: lane (g, li) supplies column li, the same k-slots;
//      C/D: lane (g, li) holds rows 4g..4g+3 of column li.
//    A and B use the same lane->k assignment, so any consistent mapping of
//    k-slots to physical indices is a valid contraction; the kernels use
//    this to feed accumulator tiles straight back in as B operands.
//  * bf16 tiles use v_mfma_f32_16x16x32_bf16 (8 k-slots per lane, K = 32);
//    fp32 tiles use v_mfma_f32_16x16x4_f32 (1 k-slot per lane, K = 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte vector

constexpr int kThreads = 256;
constexpr int kWaves = 4;

enum PhiKind { PHI_ELU1 = 0, PHI_FAVOR = 1, PHI_IDENTITY = 2 };

// ------------------------------------------------------------------ MFMA

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename OP> struct Op;
template <> struct Op<bf16> {
  using frag = bf16x8;
  static constexpr int K = 32;      // contraction length of one MFMA
  static constexpr int PL = 8;      // k-slots per lane
};
template <> struct Op<float> {
  using frag = float;
  static constexpr int K = 4;
  static constexpr int PL = 1;
};

// Fragment of PL consecutive operand elements (16-byte aligned for bf16).
template <typename OP>
__device__ __forceinline__ typename Op<OP>::frag load_frag(const OP* p) {
  return *reinterpret_cast<const typename Op<OP>::frag*>(p);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ------------------------------------------------------------------ conversions

// Elements held by one 16-byte vector.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> { static constexpr int N = 8; };
template <> struct Vec16<float> { static constexpr int N = 4; };

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <typename T>
__device__ __forceinline__ void unpack16(const u32x4& u, float* f);
template <>
__device__ __forceinline__ void unpack16<bf16>(const u32x4& u, float* f) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
  f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}
template <>
__device__ __forceinline__ void unpack16<float>(const u32x4& u, float* f) {
  f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
}

// Round-to-nearest-even float -> OP (hardware convert for bf16).
template <typename OP> __device__ __forceinline__ OP to_op(float x);
template <> __device__ __forceinline__ bf16 to_op<bf16>(float x) { return static_cast<bf16>(x); }
template <> __device__ __forceinline__ float to_op<float>(float x) { return x; }

template <typename OP> __device__ __forceinline__ float from_op(OP x);
template <> __device__ __forceinline__ float from_op<bf16>(bf16 x) { return static_cast<float>(x); }
template <> __device__ __forceinline__ float from_op<float>(float x) { return x; }

// Value after a round trip through OP (what an MFMA operand really holds).
template <typename OP> __device__ __forceinline__ float round_op(float x) { return from_op<OP>(to_op<OP>(x)); }

typedef float f32x8 __attribute__((ext_vector_type(8)));

// Round-to-nearest-even conversions of whole vectors (v_cvt_pk_bf16_f32:
// two elements per instruction).
__device__ __forceinline__ bf16x8 cvt_bf16x8(const float* f) {
  const f32x8 v = {f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]};
  return __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ bf16x4 cvt_bf16x4(f32x4 v) { return __builtin_convertvector(v, bf16x4); }

// Pack 16 bytes worth of floats (8 for bf16, 4 for fp32) into one vector.
template <typename OP>
__device__ __forceinline__ u32x4 pack16(const float* f);
template <>
__device__ __forceinline__ u32x4 pack16<bf16>(const float* f) {
  return __builtin_bit_cast(u32x4, cvt_bf16x8(f));
}
template <>
__device__ __forceinline__ u32x4 pack16<float>(const float* f) {
  return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
}

// ------------------------------------------------------------------ feature maps

// Pointwise feature maps.  ELU(x)+1 with alpha = 1 is x + 1 for x > 0 and
// e^x otherwise, evaluated as max(x + 1, e^-|x|): for x <= 0, e^x >= 1 + x
// (convexity), so the max is e^x; for x > 0, e^-x < 1 < x + 1.  Four VALU
// operations (scale with the -|.| input modifiers, exp2, add, max) instead
// of a compare and a select around both branches, and the exponential only
// ever sees non-positive arguments.  Near x = 0 the two sides agree to
// within the exp2's rounding, below the bf16 operands' resolution.
template <int PHI>
__device__ __forceinline__ float phi_pointwise(float x) {
  if constexpr (PHI == PHI_ELU1) {
    return __builtin_fmaxf(x + 1.f, __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * 1.4426950408889634f));
  } else {
    return x;
  }
}

// ------------------------------------------------------------------ wave helpers

// Index of this wave in its workgroup, as a wave-uniform (scalar) value, so
// that branches on it are scalar branches rather than exec-mask regions.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float xor_sum16_32(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace la
