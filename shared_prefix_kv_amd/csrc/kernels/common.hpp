// Device-side types shared by the gfx950 kernels: storage conversions and the
// per-dtype MFMA fragment traits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jev {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16-byte register / LDS staging unit (a native vector, so copies stay in registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 is stored as its 16-bit pattern.
struct bf16s {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16s v) { return __uint_as_float(uint32_t(v.bits) << 16); }

// float -> storage, round to nearest even.
template <typename T>
__device__ __forceinline__ T from_f32(float f);
template <>
__device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <>
__device__ __forceinline__ bf16s from_f32<bf16s>(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return bf16s{uint16_t(u >> 16)};
}

// MFMA 32x32 traits.  A operand (32 x KSTEP) lane l holds row l%32, k elements
// [KL*(l/32), KL*(l/32)+KL); B operand (KSTEP x 32) lane l holds column l%32
// and the same k range; C (32 x 32 fp32) lane l holds column l%32, rows
// 8*(r/4) + 4*(l/32) + r%4 for r in [0,16).
template <typename T>
struct Mfma;

template <>
struct Mfma<bf16s> {
  static constexpr int KL = 8;      // k elements per lane per operand
  static constexpr int KSTEP = 16;  // k per instruction
  typedef bf16x8 frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // 16 bytes at p (8 consecutive k elements)
  __device__ static __forceinline__ frag load(const void* p) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const u32x4*>(p));
  }
};

template <>
struct Mfma<float> {
  static constexpr int KL = 1;
  static constexpr int KSTEP = 2;
  typedef float frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag load(const void* p) {
    return *reinterpret_cast<const float*>(p);
  }
};

// Max / sum of v over lanes i and i ^ 32, with one VALU lane swap (no LDS
// permute): the swap of a value with itself returns, in every lane, the pair
// (lane i mod 32, lane i mod 32 + 32) in that order.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace dev
}  // namespace jev
