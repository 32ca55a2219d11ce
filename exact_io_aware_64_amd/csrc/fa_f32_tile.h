// fp32 tiles in LDS and the fp32 matrix instruction, shared by the fp32
// forward and backward kernels, for head dimension D = 32, 64 or 128.
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
// A tile is 64 rows of D floats (D / 4 16-byte chunks per row); logical
// chunk c of row j is stored at physical chunk c ^ (j % S), S = min(D / 4,
// 16), so that the 16-byte row reads (32 rows, one chunk column) and the
// 4-byte column reads (one row per wave half, 32 consecutive columns) spread
// over the banks.  XOR with j % 16 keeps a chunk inside its aligned group of
// 16, so at D = 128 a chunk c >= 16 sits 64 floats after chunk c - 16 of the
// same row: the kernels keep the offsets of the first 64 columns in
// registers and reach the rest with an immediate.
#pragma once

#include "fa_device.h"

namespace fa {
namespace f32t {

template <int D>
struct Geo {
  static_assert(D == 32 || D == 64 || D == 128, "head dimension 32, 64 or 128");
  static constexpr int kTileF = 64 * D;                     // floats per LDS tile
  static constexpr int kCpr = D / 4;                        // 16-byte chunks per row
  static constexpr int kSwz = (kCpr < 16 ? kCpr : 16) - 1;  // swizzle mask
  static constexpr int kNG = D / 8;                         // row-read groups
  static constexpr int kNDB = D / 32;                       // 32-column blocks
  static constexpr int kRowOffs = kNG < 8 ? kNG : 8;        // row offsets kept
  static constexpr int kColDB = kNDB < 2 ? kNDB : 2;        // column blocks kept
};

// Float offset of (row, col) inside a swizzled fp32 tile.
template <int D>
__device__ __forceinline__ int foff(int row, int col) {
  return row * D + (((col >> 2) ^ (row & Geo<D>::kSwz)) << 2) + (col & 3);
}

// Copies rows row0 .. row0 + 63 of a slice (byte row stride stride_b) into a
// swizzled tile straight from memory.  One buffer_load_dwordx4 ... lds moves
// 1 KiB, 256 / D rows (lane l to row l / (D / 4), physical chunk
// l % (D / 4)); the W waves of the workgroup share the D / 4 copies of a
// tile.  Rows past the slice read as zeros.  Completion is tracked by the
// wave's vmcnt.
template <int D, int W>
__device__ __forceinline__ void stage(__amdgpu_buffer_rsrc_t rs, int row0, int stride_b,
                                      float* tile, int w, int lane) {
  using G = Geo<D>;
  constexpr int kRpi = 256 / D;  // rows per copy
  static_assert((D / 4) % W == 0, "copies per wave");
#pragma unroll
  for (int u = 0; u < D / 4 / W; ++u) {
    const int first = (u * W + w) * kRpi;
    const int row = first + lane / G::kCpr;
    const int voff = row * stride_b + (((lane % G::kCpr) ^ (row & G::kSwz)) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_void_t*)(tile + first * D), 16, voff,
        __builtin_amdgcn_readfirstlane(row0 * stride_b), 0, 0);
  }
}

__device__ __forceinline__ f32x16 mfma(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Per-lane float offsets of the two kinds of LDS reads of a tile: the row
// read of group g (row r, chunk 2 g + hl; a further 32-row block adds 32 D)
// and the column reads of rows 8 h + 4 hl + i at column 32 db + r (a further
// 16-row block adds 16 D, which keeps the swizzle).  Groups g >= 8 and column
// blocks db >= 2 (D = 128) add 64 to the offset of g - 8 or db - 2.
template <int D>
struct Offsets {
  using G = Geo<D>;
  int row[G::kRowOffs], col[8 * G::kColDB];
  __device__ __forceinline__ void init(int r, int hl) {
#pragma unroll
    for (int g = 0; g < G::kRowOffs; ++g) row[g] = foff<D>(r, 8 * g + 4 * hl);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int db = 0; db < G::kColDB; ++db)
          col[(4 * h + i) * G::kColDB + db] = foff<D>(8 * h + 4 * hl + i, 32 * db + r);
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
    for (int g = 0; g < G::kRowOffs; ++g) __asm__ volatile("" : "+v"(row[g]));
#pragma unroll
    for (int x = 0; x < 8 * G::kColDB; ++x) __asm__ volatile("" : "+v"(col[x]));
  }
  __device__ __forceinline__ int rowoff(int g) const { return row[g % 8] + 64 * (g / 8); }
  __device__ __forceinline__ int coloff(int h, int i, int db) const {
    return col[(4 * h + i) * G::kColDB + db % 2] + 64 * (db / 2);
  }
};

// acc[db] += (T^T X) over the 32 rows of block `blk` (0, 1) of a 64-row
// tile T, for the output rows (columns of T) 32 db .. 32 db + 31: the A
// operand is T's column 32 db + r at row 32 blk + 8 (e / 4) + 4 hl + e % 4,
// the B operand element e of x (X's row of that index in the lane's
// column).  The column reads of a group of four steps are issued one group
// ahead.
template <int D>
__device__ __forceinline__ void col_product(const float* tile, const Offsets<D>& of, int blk,
                                            const f32x16& x, f32x16 (&acc)[D / 32]) {
  constexpr int NDB = D / 32;
  auto cread = [&](int j, float (&dst)[4 * NDB]) FA_INLINE {  // step group j = e / 4
    const int rb = 16 * (2 * blk + (j >> 1)), h = j & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int db = 0; db < NDB; ++db) dst[NDB * i + db] = tile[D * rb + of.coloff(h, i, db)];
  };
  float nx[4 * NDB], cu[4 * NDB];
  cread(0, nx);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int x2 = 0; x2 < 4 * NDB; ++x2) cu[x2] = nx[x2];
    if (j + 1 < 4) cread(j + 1, nx);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = mfma(cu[NDB * i + db], x[4 * j + i], acc[db]);
    FA_FENCE();
  }
}

// Returns T_blk R^T for the 32 rows of block blk of a tile and the 32
// register rows whose fragments are in f (f[4 g + i] = element
// 8 g + 4 hl + i of the lane's row): A is the tile's row, B the fragment.
// Each row read (four steps) is issued one group ahead.
template <int D>
__device__ __forceinline__ f32x16 row_product(const float* tile, const Offsets<D>& of, int blk,
                                              const float (&f)[D / 2]) {
  constexpr int NG = D / 8;
  f32x16 acc = zero16();
  auto rread = [&](int g) FA_INLINE {
    return *reinterpret_cast<const f32x4*>(tile + 32 * D * blk + of.rowoff(g));
  };
  f32x4 nx = rread(0);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const f32x4 cu = nx;
    if (g + 1 < NG) nx = rread(g + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mfma(cu[i], f[4 * g + i], acc);
    FA_FENCE();
  }
  return acc;
}

// Loads the lane's D / 2 fragment elements of row `row` (elements
// 8 g + 4 hl + i) through a buffer resource; rows past the end read zeros.
template <int D>
__device__ __forceinline__ void load_frag(__amdgpu_buffer_rsrc_t rs, int row, int stride_b,
                                          int hl, float (&f)[D / 2]) {
  const int off = row * stride_b + 16 * hl;
#pragma unroll
  for (int g = 0; g < D / 8; ++g) {
    const f32x4 x =
        __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32 * g, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) f[4 * g + i] = x[i];
  }
}

// Stores the lane's part of a 32-row block of output rows held transposed
// in acc (element e of block db: column 32 db + 8 (e / 4) + 4 hl + e % 4 of
// row `out`), each multiplied by s, as 16-byte stores.
template <int D>
__device__ __forceinline__ void store_rows(float* out, int hl, const f32x16 (&acc)[D / 32],
                                           float s) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 v4;
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = acc[db][4 * j + i] * s;
      *reinterpret_cast<f32x4*>(out + 32 * db + 8 * j + 4 * hl) = v4;
    }
}

}  // namespace f32t
}  // namespace fa
