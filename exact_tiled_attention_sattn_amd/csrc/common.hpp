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
  // A block past the limit raises a flag (recomputed after the walk)
  // rather than being redone at once.
  static constexpr bool kRedoBlocks = false;
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
  // Large logits reach this limit often: a block past it is redone at once.
  static constexpr bool kRedoBlocks = true;
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

// Writes a wave's 32 x D output tile, held in the 32x32x16 MFMA accumulator
// layout (lane l owns row l % 32; acc[db][4*g4 + e] is column
// db*32 + 8*g4 + 4*(l / 32) + e), times `mul`, rounded once, as whole rows.
// Stored straight from that layout, one instruction would write 8 bytes into
// each of 32 rows (32 partial cache lines). Instead the wave writes its rows
// into its own LDS slice `st` (32 * D elements; 16-byte chunk c of row r at
// chunk c ^ (r mod D/8), which spreads a column of chunks over the banks),
// then stores 16-byte lanes covering 64 / (D/8) whole rows per instruction,
// nontemporal. Row r (only r < rows) goes to dst + r * rs. The caller makes
// sure no other wave still reads `st`.
template <class E, int D>
__device__ __forceinline__ void store_tile_rows(const f32x16 (&acc)[D / 32], float mul, uint16_t* st,
                                                uint16_t* dst, int64_t rs, int rows) {
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per store instruction
  int lane = threadIdx.x & 63;
  // the lane-dependent offsets are formed here, not hoisted into the
  // caller's main loop, where they would hold registers for its whole walk
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int c = db * 4 + g4;
      const u32x2 v = {E::pack2(acc[db][g4 * 4 + 0] * mul, acc[db][g4 * 4 + 1] * mul),
                       E::pack2(acc[db][g4 * 4 + 2] * mul, acc[db][g4 * 4 + 3] * mul)};
      *(u32x2*)(st + l32 * D + ((c ^ (l32 & (CPR - 1))) * 8) + 4 * hf) = v;
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's rows are in LDS
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int r = it * RPI + lane / CPR;
    const int c = lane % CPR;
    const u32x4 val = *(const u32x4*)(st + r * D + ((c ^ (r & (CPR - 1))) * 8));
    if (r < rows) __builtin_nontemporal_store(val, (u32x4*)(dst + (int64_t)r * rs + c * 8));
  }
}

}  // namespace sattn
