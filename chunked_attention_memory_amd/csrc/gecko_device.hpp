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
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

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

// acc + lo + hi of a word holding two bf16 values (v_dot2 against (1, 1)).
__device__ __forceinline__ float sum2_bf16(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u), acc,
                                         false);
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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Sum / max of a value with the same lane of the other 32-lane half.
__device__ __forceinline__ float other_half_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float other_half_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n only:
// vmcnt in bits 3:0 and 15:14, expcnt (bits 6:4) and lgkmcnt (bits 11:8) at
// their maxima (no wait).
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// The waits use the builtin, not inline asm: the compiler's own wait
// insertion then knows the loads are done and adds no wait of its own.
// The empty asm with a memory clobber keeps memory accesses after the wait.
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  asm volatile("" ::: "memory");
}
// Workgroup barrier without the memory fence of __syncthreads, whose release
// side waits for every outstanding global load of the wave (loads prefetching
// later tiles included). The caller first makes what the other waves will
// read complete: its LDS-writing loads with wait_vmem / wait_vmem_leave, its
// LDS stores with the lgkmcnt wait here. The empty asm statements with a
// memory clobber keep the compiler from moving memory accesses across.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// wait until at most N vector-memory loads of this wave are in flight (they
// complete in issue order, so the N most recent ones may still be pending)
template <int N>
__device__ __forceinline__ void wait_vmem_leave() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(N));
  asm volatile("" ::: "memory");
}

// Copy rows [row0, row0 + rows_in_tile) of a row-major bf16 matrix with `width`
// columns into LDS with buffer loads that write LDS directly (lane l of a
// load lands at 16 l bytes past the load's LDS base, held in M0); rows at or
// past n read as zero (the buffer's size ends at row n). Load i of wave w
// fills the 1 KiB piece nwaves i + w of the tile; off[i] is the byte offset,
// within the rows starting at row0, that this lane fetches for load i.
//
// The loads are issued from inline asm so that the compiler does not track
// them: it cannot tell which LDS variable they write and would otherwise wait
// for all of them before LDS reads of other stages. Every caller waits for
// them itself (wait_vmem / wait_vmem_leave, then a barrier) before any wave
// reads what they wrote. They have no destination register; M0 is set by the
// compiler through the input constraint, and the s_nop covers the M0 -> LDS
// load hazard. A plain __device__ function on purpose: kernels' lambdas are
// also compiled for the host.
//
// A tile of fewer 1 KiB pieces than nwaves * nloads (npieces, when positive)
// is covered with pieces taken modulo npieces: several waves then load the
// same piece into the same place (the same bytes), and every wave still
// issues nloads loads, so that the waits that count them stay uniform.
// off[i] must be computed from the same piece index.
__device__ __forceinline__ int stage_piece(int nwaves, int w, int i, int npieces) {
  const int p = nwaves * i + w;
  return npieces > 0 ? p % npieces : p;
}
__device__ __forceinline__ void stage_rows(const uint16_t* base, int row0, int n, int width, char* lds_tile,
                                           int nwaves, int w, const uint32_t* off, int nloads, int npieces = 0) {
  const uint32_t rows = (uint32_t)(n > row0 ? n - row0 : 0);
  const uint64_t addr = (uint64_t)(uintptr_t)(base + (size_t)row0 * width);
  i32x4 rs;  // buffer resource: base address, stride 0, size in bytes, raw-buffer flags
  rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
  rs[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(addr >> 32) & 0xFFFFu));
  rs[2] = __builtin_amdgcn_readfirstlane((int)(rows * (uint32_t)width * 2u));
  rs[3] = 0x00020000;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_tile;
#pragma unroll
  for (int i = 0; i < nloads; ++i) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(stage_piece(nwaves, w, i, npieces) * 1024));
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off[i]), "s"(rs), "{m0}"(m0)
                 : "memory");
  }
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16): in each 16-lane group,
// source lane s addresses 4 consecutive bf16 values M[s][0..3]; lane i
// receives M[4 j + i / 4][i % 4] for j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr(const char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}

// XOR swizzle of the 16-byte chunks of a staged row-major V row (dv values),
// for transpose reads of 4 rows x 32 columns (32 lanes per pass, 64 banks).
// It depends on the row mod 4 only. Rows of 64 bytes (dv = 32) hold 4 chunks.
template <int DV>
__device__ __forceinline__ int vswz(int r) {
  if constexpr (DV >= 128) return (r & 3) << 2;
  if constexpr (DV == 64) return ((r >> 1) & 1) << 2;
  return r & 3;
}

}  // namespace gecko
