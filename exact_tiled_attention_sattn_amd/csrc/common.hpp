// Device-side helpers shared by the sattn kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element traits: the 16-bit storage type, its 32x32x16 MFMA, its
// round-to-nearest-even packing of two fp32 values and the exact unpacking.
struct Bf16 {
  // Largest per-tile sum of exps the fixed-reference update accepts (bf16
  // shares fp32's exponent range, so only the fp32 sums bound it).
  static constexpr float kFastLimit = 18446744073709551616.0f;  // 2^64
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  // the two values of a packed word, exactly, as fp32
  static __device__ __forceinline__ float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
};

struct F16 {
  // The rounded P must stay below fp16's largest finite value, 65504.
  static constexpr float kFastLimit = 32768.0f;  // 2^15
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2 r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
  static __device__ __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Low 16-bit halves of two words -> one word (lo from a, hi from b).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
// High 16-bit halves of two words -> one word (lo from a, hi from b).
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Value of `x` held by lane (lane ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

}  // namespace sattn
