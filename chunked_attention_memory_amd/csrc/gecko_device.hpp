// Device-side helpers shared by the gfx950 kernels: bf16 packing, the
// 32x32x16 bf16 MFMA wrapper and the row permutation used to make MFMA
// accumulator rows contiguous per lane.
//
// MFMA 32x32x16 (bf16 in, fp32 accumulate) operand layout, per 64-lane wave:
//   A (32 x 16): lane l holds row (l & 31), k-slice [8 (l >> 5), 8 (l >> 5) + 8)
//   B (16 x 32): lane l holds col (l & 31), the same k-slice
//   C (32 x 32): lane l holds col (l & 31); register r holds row
//                8 (r >> 2) + 4 (l >> 5) + (r & 3)
// The hardware's own order inside a k-slice is the same for A and B, so the
// contraction is correct whatever it is.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gecko {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Round two floats to bf16 (round to nearest even) and pack (a in the low half).
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Swap bits 2 and 3 of a row index inside a 32-row block. If lane l of an
// MFMA A operand loads logical row perm_row(l & 31), then accumulator register
// r of a lane in half g holds logical row (r & 7) + 8 g + 16 (r >> 3): eight
// consecutive rows per half-register-file. It is its own inverse.
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// 8x8 transpose of bf16 held as 8 rows of 4 packed words: out[c] word j holds
// (in[2j] col c, in[2j+1] col c).
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int c2 = 0; c2 < 4; ++c2) {      // column pair (2 c2, 2 c2 + 1)
#pragma unroll
    for (int j = 0; j < 4; ++j) {       // output word j: rows 2j, 2j + 1
      const uint32_t a = in[2 * j][c2];
      const uint32_t b = in[2 * j + 1][c2];
      out[2 * c2][j] = __builtin_amdgcn_perm(b, a, 0x05040100u);      // low halves
      out[2 * c2 + 1][j] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // high halves
    }
  }
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace gecko
