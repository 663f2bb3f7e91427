// Device helpers of the backward kernels: LDS tile layout and the two MFMA
// operand reads from it.
//
// Tiles are staged row-major (rows of W bf16, W = 128 or 256) with the
// 16-byte chunks of row r XOR-swizzled by sw16(r). Two reads are used:
//  * lds_row: 16 bytes of one row (an operand whose rows, or columns, are the
//    tile's rows). Sixteen consecutive rows read at the same logical chunk hit
//    sixteen different bank groups.
//  * lds_tr: the transpose read (ds_read_b64_tr_b16) of 4 rows x 32 columns
//    per 32 lanes, for an operand whose k index runs along the tile's rows.
//    Four rows r0 + [0, 4) (r0 = 0 mod 4) at four consecutive chunks land on
//    sixteen different bank groups, since sw16 moves bits 0-1 of the row into
//    bits 2-3 of the chunk.
//
// Row order of accumulators: both reads give lane l the row (or column)
// perm_row(l & 31) of its 32-block. An MFMA whose A operand rows come in that
// order leaves register r of a lane in half g holding logical row
// (r & 7) + 8 g + 16 (r >> 3), which is the k order of a B operand (lane half g
// holds k = 8 g + [0, 8) of each 16-step). So accumulators feed the next MFMA
// as B operands without a shuffle, and line up element by element with
// per-lane vectors loaded in B-operand order.
#pragma once

#include "gecko_device.hpp"

namespace gecko {

__device__ __forceinline__ int sw16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// 16 bytes (k = 8 chunk + [0, 8)) of row `row` of a staged tile with W columns
template <int W>
__device__ __forceinline__ u32x4 lds_row(const char* t, int row, int chunk) {
  return *reinterpret_cast<const u32x4*>(t + row * (W * 2) + 16 * (chunk ^ sw16(row)));
}

// Operand of lane l: row (A) or column (B) col0 + perm_row(l & 31) of the
// transposed tile, k = r0 + 8 g + [0, 8) (tile rows). In each 16-lane group
// source lane s points at tile row r0 + 8 g + s / 4 (+ 4 for the second read)
// and 4 columns starting at col0 + 16 (group % 2) + 4 swap2(s % 4); lane i of
// the group then receives column col0 + 16 (group % 2) + perm_row(i) of the
// four rows (ds_read_b64_tr_b16: lane i gets element i % 4 of source lanes
// 4 j + i / 4, j = 0..3).
// kPerm = false gives column col0 + (l & 31) instead (plain accumulator row
// order, for results kept in the memory scan's layout).
template <int W, bool kPerm = true>
__device__ __forceinline__ u32x4 lds_tr(const char* t, int r0, int col0, int lane) {
  const int s = lane & 15, grp = (lane >> 4) & 1, g = lane >> 5;
  const int a = s & 3;
  const int col = col0 + 16 * grp + 4 * (kPerm ? (((a & 1) << 1) | (a >> 1)) : a);
  const int r = r0 + 8 * g + (s >> 2);
  const u32x2 lo = lds_read_tr(t + r * (W * 2) + 16 * ((col >> 3) ^ sw16(r)) + 2 * (col & 7));
  const u32x2 hi = lds_read_tr(t + (r + 4) * (W * 2) + 16 * ((col >> 3) ^ sw16(r + 4)) + 2 * (col & 7));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// The same reads with the lane-dependent part of the address computed once.
// For a block of rows starting at a multiple of 16, sw16 of a row depends on
// the lane only, and the swizzle splits into a constant XOR on the high chunk
// bits and a fixed low part, so a read costs one XOR and one add.
//
// RowReader: lds_row(t, row0 + perm_row(l & 31), 2 ks + g) for row0 = 0 mod 16.
template <int W>
struct RowReader {
  int base;  // perm_row(lq) W 2 + 16 ((g ^ sw) & 1)
  int swh;   // sw16(perm_row(lq)) & 14
  __device__ __forceinline__ void init(int lane) {
    const int r = perm_row(lane & 31), g = lane >> 5, sw = sw16(r);
    base = r * (W * 2) + 16 * ((g ^ sw) & 1);
    swh = sw & 14;
  }
  __device__ __forceinline__ u32x4 read(const char* t, int row0, int ks) const {
    return *reinterpret_cast<const u32x4*>(t + row0 * (W * 2) + base + 16 * ((2 * ks) ^ swh));
  }
};

// TrReader: lds_tr<W, kPerm>(t, r0, 32 blk, lane) for r0 = 0 mod 16.
template <int W, bool kPerm = true>
struct TrReader {
  int base0, base1;  // rows 8 g + s / 4 (+ 4): row offset, low chunk bits, byte within the chunk
  int swh0, swh1;    // high chunk bits of the two rows' swizzles
  __device__ __forceinline__ void init(int lane) {
    const int s = lane & 15, grp = (lane >> 4) & 1, g = lane >> 5, a = s & 3;
    const int p2 = kPerm ? (((a & 1) << 1) | (a >> 1)) : a;
    const int cl = 2 * grp + (p2 >> 1), eoff = 8 * (p2 & 1);
    const int r0 = 8 * g + (s >> 2), r1 = r0 + 4;
    const int sw0 = sw16(r0), sw1 = sw16(r1);
    base0 = r0 * (W * 2) + 16 * (cl ^ (sw0 & 3)) + eoff;
    base1 = r1 * (W * 2) + 16 * (cl ^ (sw1 & 3)) + eoff;
    swh0 = sw0 & 12;
    swh1 = sw1 & 12;
  }
  __device__ __forceinline__ u32x4 read(const char* t, int r0, int blk) const {
    const char* p = t + r0 * (W * 2);
    const u32x2 lo = lds_read_tr(p + base0 + 16 * ((4 * blk) ^ swh0));
    const u32x2 hi = lds_read_tr(p + base1 + 16 * ((4 * blk) ^ swh1));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
};

// Source byte offsets for stage_rows: LDS chunk P = (nw i + w) 64 + lane of
// load i is physical chunk P % (W / 8) of tile row P / (W / 8), which holds
// logical chunk (P % (W / 8)) ^ sw16(row).
template <int W, int NL>
__device__ __forceinline__ void stage_offsets(uint32_t (&off)[NL], int nw, int w, int lane) {
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int P = (nw * i + w) * 64 + lane;
    const int r = P / (W / 8), p = P % (W / 8);
    off[i] = (uint32_t)(r * W + 8 * (p ^ sw16(r))) * 2u;
  }
}

__device__ __forceinline__ u32x4 pack8(const float* x) {
  return u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
}

__device__ __forceinline__ void unpack8(u32x4 w, float* x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf_lo(w[j]);
    x[2 * j + 1] = bf_hi(w[j]);
  }
}

// flip the sign of 8 packed bf16 values (exact)
__device__ __forceinline__ u32x4 neg8(u32x4 w) {
  return u32x4{w[0] ^ 0x80008000u, w[1] ^ 0x80008000u, w[2] ^ 0x80008000u, w[3] ^ 0x80008000u};
}

}  // namespace gecko
