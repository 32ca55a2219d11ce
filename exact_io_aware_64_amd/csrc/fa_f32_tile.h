// fp32 tiles in LDS and the fp32 matrix instruction, shared by the fp32
// forward and backward kernels.
//
// A 32x32x2 fp32 MFMA contracts over two indices, one per wave half: lane
// (r, hl) (r = lane % 32, hl = lane / 32) supplies element (r, hl) of the A
// operand and (hl, r) of B, and its accumulator holds column r, rows
// 8 (v / 4) + 4 hl + v % 4 (v = 0..15).  Any pairing of the contraction
// indices works as long as A and B use the same one; the kernels pair them
// so that no lane needs another lane's data:
//   * a product whose contraction runs over the head dimension contracts,
//     at step s, index 8 (s / 4) + 4 hl + s % 4: four steps of a lane come
//     from one 16-byte read of a tile row and four registers of its own row;
//   * a product whose contraction runs over the rows of a tile (keys or
//     queries) contracts, at step e, row 8 (e / 4) + 4 hl + e % 4 -- the
//     row held in element e of the lane's accumulator column, so that a
//     probability (or dS) feeds the B operand as it stands and A is a 4-byte
//     read of a tile column.
// A tile is 64 rows of 64 floats (256 bytes, sixteen 16-byte chunks); logical
// chunk c of row j is stored at physical chunk c ^ (j % 16), so that the
// 16-byte row reads (32 rows, one chunk column) and the 4-byte column reads
// (one row per wave half, 32 consecutive columns) meet distinct banks.
#pragma once

#include "fa_device.h"

namespace fa {
namespace f32t {

constexpr int kD = 64;           // head dimension
constexpr int kTileF = 64 * 64;  // floats per LDS tile

// Float offset of (row, col) inside a swizzled fp32 tile.
__device__ __forceinline__ int foff(int row, int col) {
  return row * 64 + (((col >> 2) ^ (row & 15)) << 2) + (col & 3);
}

// Copies rows row0 .. row0 + 63 of a slice (byte row stride stride_b) into a
// swizzled tile straight from memory: one buffer_load_dwordx4 ... lds moves
// 4 rows (lane l to row l / 16, physical chunk l % 16), and each of the 4
// waves of the workgroup issues 4 of them.  Rows past the slice read as
// zeros.  Completion is tracked by the wave's vmcnt.
__device__ __forceinline__ void stage(__amdgpu_buffer_rsrc_t rs, int row0, int stride_b,
                                      float* tile, int w, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 16 * u + 4 * w + (lane >> 4);
    const int voff = row * stride_b + (((lane & 15) ^ (row & 15)) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_void_t*)(tile + (16 * u + 4 * w) * 64), 16, voff,
        __builtin_amdgcn_readfirstlane(row0 * stride_b), 0, 0);
  }
}

__device__ __forceinline__ f32x16 mfma(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Per-lane float offsets of the two kinds of LDS reads of a tile: the row
// read of group g (row r, chunk 2 g + hl; a further 32-row block adds 2048)
// and the column reads of rows 8 h + 4 hl + i at column 32 db + r (entry
// 8 h + 2 i + db; a further 16-row block adds 1024, which keeps the swizzle).
struct Offsets {
  int row[8], col[16];
  __device__ __forceinline__ void init(int r, int hl) {
#pragma unroll
    for (int g = 0; g < 8; ++g) row[g] = foff(r, 8 * g + 4 * hl);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int db = 0; db < 2; ++db) col[8 * h + 2 * i + db] = foff(8 * h + 4 * hl + i, 32 * db + r);
  }
  // Recomputed from an opaque copy of the lane index, for kernels that
  // cannot keep the offsets live across their tile loop.
  __device__ __forceinline__ void init_here(int lane) {
    __asm__ volatile("" : "+v"(lane));
    init(lane & 31, lane >> 5);
  }
  // Fresh copies for the next tile: otherwise the compiler keeps one
  // register per buffer and offset live across the tile loop.
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int g = 0; g < 8; ++g) __asm__ volatile("" : "+v"(row[g]));
#pragma unroll
    for (int x = 0; x < 16; ++x) __asm__ volatile("" : "+v"(col[x]));
  }
};

// acc[db] += (T^T X) over the 32 rows of block `blk` (0, 1) of a 64-row
// tile T, for the output rows (columns of T) 32 db .. 32 db + 31: the A
// operand is T's column 32 db + r at row 32 blk + 8 (e / 4) + 4 hl + e % 4,
// the B operand element e of x (X's row of that index in the lane's
// column).  The column reads of a group of four steps are issued one group
// ahead.
__device__ __forceinline__ void col_product(const float* tile, const Offsets& of, int blk,
                                            const f32x16& x, f32x16 (&acc)[2]) {
  auto cread = [&](int j, float (&dst)[8]) FA_INLINE {  // step group j = e / 4
    const int rb = 16 * (2 * blk + (j >> 1)), h = j & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int db = 0; db < 2; ++db) dst[2 * i + db] = tile[64 * rb + of.col[8 * h + 2 * i + db]];
  };
  float nx[8], cu[8];
  cread(0, nx);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int x2 = 0; x2 < 8; ++x2) cu[x2] = nx[x2];
    if (j + 1 < 4) cread(j + 1, nx);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int db = 0; db < 2; ++db) acc[db] = mfma(cu[2 * i + db], x[4 * j + i], acc[db]);
    FA_FENCE();
  }
}

// Returns T_blk R^T for the 32 rows of block blk of a tile and the 32
// register rows whose fragments are in f (f[4 g + i] = element
// 8 g + 4 hl + i of the lane's row): A is the tile's row, B the fragment.
// Each row read (four steps) is issued one group ahead.
__device__ __forceinline__ f32x16 row_product(const float* tile, const Offsets& of, int blk,
                                              const float (&f)[32]) {
  f32x16 acc = zero16();
  auto rread = [&](int g) FA_INLINE {
    return *reinterpret_cast<const f32x4*>(tile + 2048 * blk + of.row[g]);
  };
  f32x4 nx = rread(0);
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const f32x4 cu = nx;
    if (g + 1 < 8) nx = rread(g + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mfma(cu[i], f[4 * g + i], acc);
    FA_FENCE();
  }
  return acc;
}

// Loads the lane's 32 fragment elements of row `row` (elements
// 8 g + 4 hl + i) through a buffer resource; rows past the end read zeros.
__device__ __forceinline__ void load_frag(__amdgpu_buffer_rsrc_t rs, int row, int stride_b,
                                          int hl, float (&f)[32]) {
  const int off = row * stride_b + 16 * hl;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const f32x4 x =
        __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32 * g, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) f[4 * g + i] = x[i];
  }
}

}  // namespace f32t
}  // namespace fa
