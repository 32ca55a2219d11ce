// Device-side building blocks for the gfx950 attention kernels: MFMA
// fragment types, wave-half exchange, LDS tile staging and the kept-tile list.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kInf = __builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  // D[32x32] += A[32x16] * B[16x32].  Lane l supplies row (l % 32) of A and
  // column (l % 32) of B, both at contraction slots 8*(l/32) .. 8*(l/32)+7, and
  // holds D[8*(e/4) + 4*(l/32) + e%4][l % 32] in element e.
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Max / sum of x over lanes l and l ^ 32 (the two halves of a wave hold the
// two halves of one query's keys).
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                            false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                            false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Elements [off, off+8) of an accumulator, rounded to bf16 (nearest-even).
__device__ __forceinline__ bf16x8 pack8(const f32x16& v, int off) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)v[off + i];
  return r;
}

// Two floats rounded to bf16 (nearest-even) and packed low, high.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// acc + sum of the 8 products x[i] * y[i] (bf16 products are exact in fp32).
__device__ __forceinline__ float dot8_bf16(bf16x8 x, bf16x8 y, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1),
                                        __builtin_shufflevector(y, y, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3),
                                        __builtin_shufflevector(y, y, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5),
                                        __builtin_shufflevector(y, y, 4, 5), acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7),
                                         __builtin_shufflevector(y, y, 6, 7), acc, false);
}

// x of the lane whose index differs in bit 0 (quad_xor1) or bit 1 (quad_xor2)
// within each group of four lanes (DPP quad permutations [1,0,3,2] and
// [2,3,0,1]).
__device__ __forceinline__ float quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

// Buffer resource over one (batch, head) slice of a tensor.  Loads through
// it take 32-bit byte offsets, and any 16-byte load that starts at or past
// `bytes` returns zeros, so rows past the end need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword3 0x00020000: the raw-buffer format word for gfx9-family GPUs.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 ldb16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Bytes spanned by rows 0..n-1 of `row` elements with row stride `ss` (elements).
__device__ __forceinline__ uint32_t slice_bytes(int n, int64_t ss, int esize, int row = 64) {
  return (uint32_t)(((int64_t)(n - 1) * ss + row) * esize);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Swizzled 64 x 64 bf16 tiles in LDS.
//
// Row r of a tile occupies 128 contiguous bytes (eight 16-byte chunks), and
// logical chunk c of row r is stored at physical chunk c ^ swz(r).  With this
// XOR pattern both reads the kernels make are free of bank conflicts on
// gfx950's LDS: 16-byte row reads (16 lanes reading one chunk column of 16
// consecutive rows) and ds_read_b64_tr_b16 transpose reads (32 lanes reading
// 4 chunks of 4 consecutive rows).  swz depends only on (r / 2) % 8, so a
// tile offset by a multiple of 16 rows keeps the same pattern.
constexpr int kTileElems = 64 * 64;

__device__ __forceinline__ int swz(int row) {
  const int p = (row >> 1) & 7;
  return (p >> 1) | ((p & 1) << 2);
}

// Element offset of (row, col) inside a swizzled tile.
__device__ __forceinline__ int toff(int row, int col) {
  return row * 64 + (((col >> 3) ^ swz(row)) << 3) + (col & 7);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Copies rows row0 .. row0+63 of one (batch, head) slice (byte row stride
// `stride_b`, buffer resource `rs`) straight from memory into the swizzled
// tile, without passing through registers: buffer_load_dwordx4 ... lds puts
// lane l's 16 bytes at the wave's LDS base + 16 l, so lane l fetches the
// logical chunk that belongs at physical chunk l % 8 of row l / 8.  In a
// workgroup of W waves, wave w copies rows 8 (w + W u) .. +7 for u < 8 / W
// (with four waves: rows 8 w .. 8 w + 7 and 8 w + 32 .. 8 w + 39, stage_row);
// those rows are 16 apart or more and the swizzle repeats every 16 rows, so
// all the wave's instructions share one per-lane offset and step the uniform
// offset.  Rows past the end of the slice read as zeros.  Completion is
// tracked by the wave's vmcnt.
__device__ __forceinline__ int stage_row(int w, int lane, int u) {
  return 8 * w + 32 * u + (lane >> 3);
}

// col_b: byte offset of the tile's first column within a row (a 64-column
// block of a wider row).
template <int W = 4>
__device__ __forceinline__ void stage_tile(__amdgpu_buffer_rsrc_t rs, int row0, int stride_b,
                                           uint16_t* tile, int w, int lane, int col_b = 0) {
  static_assert(W == 2 || W == 4 || W == 8, "a tile is copied by 2, 4 or 8 waves");
  const int row = 8 * w + (lane >> 3);
  const int voff = row * stride_b + col_b + (((lane & 7) ^ swz(row)) << 4);
#pragma unroll
  for (int u = 0; u < 8 / W; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_void_t*)(tile + (8 * w + 8 * W * u) * 64), 16, voff,
        __builtin_amdgcn_readfirstlane((row0 + 8 * W * u) * stride_b), 0, 0);
}

// 8 consecutive bf16 of a tile row (a 16-byte aligned chunk).
__device__ __forceinline__ bf16x8 tile_row8(const uint16_t* tile, int off) {
  return *reinterpret_cast<const bf16x8*>(tile + off);
}

// Row-read offset for the MFMA operand whose contraction runs along a tile
// row: lane (r, hl) reads row r (+ 32 kb, i.e. + 2048 kb elements) at columns
// 16 ks + 8 hl .. +7.
__device__ __forceinline__ int row_off(int r, int hl, int ks) { return toff(r, 16 * ks + 8 * hl); }

// Transpose-read offsets for tr_read: the A operand of a 32x32x16 MFMA whose
// contraction runs over tile ROWS 16 st .. 16 st + 15 (+ 1024 st elements)
// and whose output rows are tile columns 32 db .. 32 db + 31.  Lane (r, hl)
// receives X[16 st + 4 hl + t][32 db + r] in slots t = 0..3 and
// X[16 st + 8 + 4 hl + t][32 db + r] in slots 4..7.  Within each 16-lane
// group of a ds_read_b64_tr_b16, lane i receives element 16 t + i (t = 0..3)
// of the 64 elements the group reads, and source lane j reads 4 elements of
// row j / 4; `hi` selects the rows 8 .. 15 of the step.
__device__ __forceinline__ int tr_off(int lane, int hi, int db) {
  const int j = lane & 15, g = lane >> 4;
  return toff(8 * hi + 4 * (g >> 1) + (j >> 2), 32 * db + 16 * (g & 1) + 4 * (j & 3));
}

__device__ __forceinline__ bf16x8 tr_read(const uint16_t* tile, int off_lo, int off_hi) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off_lo));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off_hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 words_to_bf16x8(uint32_t a, uint32_t b, uint32_t c,
                                                  uint32_t d) {
  return __builtin_bit_cast(bf16x8, make_uint4(a, b, c, d));
}

#define FA_FENCE() __builtin_amdgcn_sched_barrier(0)
// Lambdas in the kernels hold per-tile code; a call left out of line would
// spill the captured state to scratch memory.
#define FA_INLINE __attribute__((always_inline))

// Workgroup ids are dealt to the 8 XCDs round robin, and within an XCD to its
// 32 CUs in order, so the k-th id of an XCD lands on CU k mod 32 in the first
// pass.  For a list ordered heaviest first, this makes CU 0 take items 0, 32,
// 64, ... of its XCD and CU 31 items 31, 63, 95, ...: every CU's share is
// skewed the same way.  snake_id turns every second run of 32 ids of an XCD
// around (items 0, 63, 64, ... on CU 0; 31, 32, 95, ... on CU 31), which
// evens out the co-resident items of a CU.  A bijection on [0, G) that keeps
// each id on its XCD and in its run of 32.
__device__ __forceinline__ int snake_id(int id, int G) {
  const int x = id & 7, k = id >> 3;
  const int cnt = (G - x + 7) >> 3;  // ids of XCD x
  const int r0 = k & ~31;
  const int len = min(32, cnt - r0);
  const int kk = ((k >> 5) & 1) ? r0 + len - 1 - (k - r0) : k;
  return kk * 8 + x;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Builds, in LDS, the list of 64-row tiles t in [t_lo, t_hi) whose mask tile
// (t / per_mask) is kept: mask entry J lives at mask[J * stride].  Called by
// all NT threads of the block (scratch holds NT / 64 ints); returns the list
// length (same in every thread).  The list is sorted ascending.
template <int NT = 256>
__device__ __forceinline__ int build_tile_list(uint16_t* list, int* scratch,
                                               const uint8_t* mask, int64_t stride,
                                               int n_mask_tiles, int per_mask, int t_lo,
                                               int t_hi) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int base = 0;
  const int j_lo = t_lo / per_mask;
  const int j_hi = (t_hi + per_mask - 1) / per_mask;  // exclusive
  for (int c0 = j_lo; c0 < j_hi; c0 += NT) {
    const int J = c0 + tid;
    int first = 0, cnt = 0;
    if (J < j_hi && J < n_mask_tiles && mask[(int64_t)J * stride] != 0) {
      first = max(J * per_mask, t_lo);
      const int last = min((J + 1) * per_mask, t_hi);
      cnt = max(0, last - first);
    }
    const int incl = wave_incl_scan(cnt);
    if (lane == 63) scratch[w] = incl;
    __syncthreads();
    int woff = 0, total = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      const int v = scratch[i];
      woff += (i < w) ? v : 0;
      total += v;
    }
    const int pos = base + woff + incl - cnt;
    for (int x = 0; x < cnt; ++x) list[pos + x] = (uint16_t)(first + x);
    base += total;
    __syncthreads();
  }
  return base;
}

// ---------------------------------------------------------------------------
// Dropout keep bytes.
//
// Every (query i, key j) pair of head slice bh gets an 8-bit uniform number
// from Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, SC'11),
// keyed by the 64-bit seed: the call with counter (j / 4, i / 4, bh, offset)
// covers the 4 x 4 block of pairs with those quotients, output word i % 4
// holding the four keys of query i in its bytes (key j % 4 in byte j % 4,
// least significant first).  A pair is kept iff its byte is below the
// threshold t, so the forward and backward passes regenerate the same mask
// without storing it.

// Rounds r0 .. r1-1 of Philox4x32 on counter x with key (k0, k1); a call
// split over several schedule slots runs its rounds in pieces.  The empty asm
// makes the key opaque, so the round keys are formed on the scalar ALU where
// they are used instead of being hoisted out of the tile loop, where the ten
// pairs would occupy twenty scalar registers for the whole kernel.
__device__ __forceinline__ void philox_rounds(uint32_t (&x)[4], uint32_t k0, uint32_t k1,
                                              int r0, int r1) {
  __asm__("" : "+s"(k0), "+s"(k1));
#pragma unroll
  for (int r = r0; r < r1; ++r) {
    const uint32_t ka = k0 + (uint32_t)r * 0x9E3779B9u;  // Weyl key schedule
    const uint32_t kb = k1 + (uint32_t)r * 0xBB67AE85u;
    const uint64_t p0 = (uint64_t)0xD2511F53u * x[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x[2];
    // three-input xor in one gfx950 bitop3 (truth table 0x96 = a ^ b ^ c)
    const uint32_t y0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), x[1], ka, 0x96);
    const uint32_t y2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), x[3], kb, 0x96);
    x[1] = (uint32_t)p1;
    x[3] = (uint32_t)p0;
    x[0] = y0;
    x[2] = y2;
  }
}

__device__ __forceinline__ uint32_t quad_xor1_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t quad_xor2_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);
}

// In every aligned group of four lanes, lane x ends with v[g] = (v[x] of lane
// g): a 4 x 4 transpose of words over the group, in two butterfly stages
// that each swap the off-diagonal halves with the partner lane.
__device__ __forceinline__ void quad_transpose(uint32_t (&v)[4], int lane) {
  const bool b0 = lane & 1, b1 = lane & 2;
#pragma unroll
  for (int w = 0; w < 4; w += 2) {
    const uint32_t got = quad_xor1_u(b0 ? v[w] : v[w + 1]);
    if (b0)
      v[w] = got;
    else
      v[w + 1] = got;
  }
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t got = quad_xor2_u(b1 ? v[w] : v[w + 2]);
    if (b1)
      v[w] = got;
    else
      v[w + 2] = got;
  }
}

// 4 x 4 byte transpose within one lane: byte y of word x <- byte x of word y.
__device__ __forceinline__ void byte_transpose(uint32_t (&v)[4]) {
  uint32_t t[4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
    t[x] = ((v[0] >> (8 * x)) & 0xFFu) | (((v[1] >> (8 * x)) & 0xFFu) << 8) |
           (((v[2] >> (8 * x)) & 0xFFu) << 16) | (((v[3] >> (8 * x)) & 0xFFu) << 24);
#pragma unroll
  for (int x = 0; x < 4; ++x) v[x] = t[x];
}

// Keep bytes of one lane for a 32 x 32 block of pairs in the MFMA
// accumulator layout, where the lane holds element 4 g + y at "row"
// 8 g + 4 hl + y of the block (g, y = 0..3) and one fixed "column":
//  * query-major (forward, dQ): the column is the lane's query qi and rows
//    are keys from kb0; the lane's call is the block (qi / 4,
//    kb0 / 4 + 2 (lane % 4) + hl), and after the quad transpose v[g] is
//    word qi % 4 of block g, i.e. the bytes of keys kb0 + 8 g + 4 hl + 0..3.
//  * key-major (dK/dV): the column is the lane's key kj and rows are queries
//    from qb0; the lane's call is the block (qb0 / 4 + 2 (lane % 4) + hl,
//    kj / 4); after the byte transpose word x holds key 4 (kj / 4) + x of
//    the block's four queries, and after the quad transpose v[g] holds
//    key kj of queries qb0 + 8 g + 4 hl + 0..3.
// Either way byte y of v[g] belongs to element 4 g + y.  The Philox rounds
// run between `start` and `finish` so that callers can spread them.
struct DropBlock {
  uint32_t v[4];
};
__device__ __forceinline__ void drop_start(DropBlock& d, uint32_t key_quad,
                                           uint32_t query_quad, uint32_t bh, uint32_t offset) {
  d.v[0] = key_quad;
  d.v[1] = query_quad;
  d.v[2] = bh;
  d.v[3] = offset;
}
template <bool KEY_MAJOR>
__device__ __forceinline__ void drop_finish(DropBlock& d, int lane) {
  if constexpr (KEY_MAJOR) byte_transpose(d.v);
  quad_transpose(d.v, lane);
}
// Is element e (0..15) of the block kept?
__device__ __forceinline__ bool drop_keep(const DropBlock& d, int e, uint32_t t) {
  return ((d.v[e >> 2] >> (8 * (e & 3))) & 0xFFu) < t;
}

}  // namespace fa
