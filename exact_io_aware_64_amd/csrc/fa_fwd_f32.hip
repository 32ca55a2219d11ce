// fp32 attention forward on the fp32 matrix cores (v_mfma_f32_32x32x2_f32).
//
// The same tiled algorithm as the bf16 forward (researchpapers.dev
// explainer, "tiling and recomputation"; suanlizi.com summary, "tiling"):
// key/value tiles of 64 rows stream through LDS against query rows held in
// registers, the scores go through an online softmax with a running maximum
// and sum, and only O and the row logsumexp L are written.  Every product is
// an fp32 product accumulated in fp32, so the results stay within ~1e-6 of
// exact: this path serves full-precision callers.
//
// One workgroup (4 waves) owns 128 query rows of one (batch, head); each wave
// owns 32 of them.  A 32x32x2 fp32 MFMA contracts over two indices, one per
// wave half: lane (r, hl) (r = lane % 32, hl = lane / 32) supplies element
// (r, k_hl) of the A operand and (k_hl, r) of B.  Any pairing of the
// contraction indices works as long as A and B use the same one, so the
// kernel picks the pairing that needs no data movement between lanes:
//   S^T = K Q^T, step s (0..31) of a 32-key block: head-dimension index
//     d(s, hl) = 8 (s / 4) + 4 hl + s % 4; lane (r, hl) holds
//     K[key r][d(s, hl)] (four steps come from one 16-byte LDS read of a K
//     row) and Q[query r][d(s, hl)] (kept in 32 registers);
//   O^T += V^T P^T, step e (0..15) of a 32-key block: key index
//     k(e, hl) = 8 (e / 4) + 4 hl + e % 4, which is exactly the key of
//     accumulator element e of the lane's S^T column, so the probability
//     feeds the B operand from the lane's own registers; A is V[k(e, hl)][d r]
//     (a 4-byte LDS read of a V column).
// The accumulators hold S^T and O^T with one query per lane column: the
// softmax needs no transposition and O rows leave as 16-byte stores.
//
// LDS tiles are 64 rows of 64 floats (256 bytes, sixteen 16-byte chunks);
// logical chunk c of row j sits at physical chunk c ^ (j % 16), so the
// 16-byte row reads (32 rows, one chunk column) and the 4-byte column reads
// (one row per wave half, 32 consecutive columns) meet distinct banks.
// Tiles are copied straight from memory into LDS, double-buffered.
//
// Masks as in the bf16 forward: key j is visible to query i iff j < the
// sequence's key length and (without the causal mask, or) j <= i + N_k - N,
// and a block mask drops whole 128 x 128 tiles before they are loaded.
// Dropout uses the same Philox4x32-10 keep bytes as the other kernels: the
// call with counter (j / 4, i / 4, b H + h, offset) gives pair (i, j) byte
// j % 4 of word i % 4.
#include "fa_device.h"

namespace fa {
namespace {

constexpr int kD = 64;             // head dimension
constexpr int kW = 4;              // waves per workgroup
constexpr int kBR = 32 * kW;       // query rows per workgroup
constexpr int kTileF = 64 * 64;    // floats per LDS tile

// Float offset of (row, col) inside a swizzled fp32 tile.
__device__ __forceinline__ int foff(int row, int col) {
  return row * 64 + ((((col >> 2) ^ (row & 15))) << 2) + (col & 3);
}

// Copies rows row0 .. row0 + 63 of a slice into a swizzled tile: one
// buffer_load_dwordx4 ... lds moves 4 rows (64 lanes x 16 bytes, lane l to
// row l / 16, physical chunk l % 16), each wave 4 such groups.
__device__ __forceinline__ void stage_f32(__amdgpu_buffer_rsrc_t rs, int row0, int stride_b,
                                          float* tile, int w, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 16 * u + 4 * w + (lane >> 4);  // rows of this instruction: 4 consecutive
    const int voff = row * stride_b + (((lane & 15) ^ (row & 15)) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_void_t*)(tile + (16 * u + 4 * w) * 64), 16, voff,
        __builtin_amdgcn_readfirstlane(row0 * stride_b), 0, 0);
  }
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Two waves per SIMD (the LDS holds two workgroups' double-buffered tiles).
template <bool DROP>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(2, 2))) void
fwd_f32_kernel(FwdArgs a, int causal) {
  __shared__ __attribute__((aligned(16))) float s_k0[kTileF];
  __shared__ __attribute__((aligned(16))) float s_v0[kTileF];
  __shared__ __attribute__((aligned(16))) float s_k1[kTileF];
  __shared__ __attribute__((aligned(16))) float s_v1[kTileF];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 31, hl = lane >> 5;
  const int BH = a.B * a.H;
  const int nqt = (a.N + kBR - 1) / kBR;
  const int qt = nqt - 1 - (int)blockIdx.x / BH;  // longest (causal) tiles first
  const int bh = (int)blockIdx.x % BH;
  const int b = bh / a.H, hh = bh % a.H;
  const int q0 = qt * kBR, qw = q0 + 32 * w, qi = qw + r;

  int kv_len = a.Nk;
  if (a.seqlens) kv_len = min(max(a.seqlens[b], 0), a.Nk);
  const int kend = causal ? max(0, min(kv_len, q0 + kBR + a.coff)) : kv_len;
  const int ntk = (kend + 63) / 64;

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(
      (const float*)a.q + b * a.sq.b + hh * a.sq.h, slice_bytes(a.N, a.sq.s, 4, kD));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(
      (const float*)a.k + b * a.sk.b + hh * a.sk.h, slice_bytes(a.Nk, a.sk.s, 4, kD));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(
      (const float*)a.v + b * a.sv.b + hh * a.sv.h, slice_bytes(a.Nk, a.sv.s, 4, kD));
  const int ssk = (int)a.sk.s * 4, ssv = (int)a.sv.s * 4;

  // Q[qi][8 m + 4 hl .. +3] for m = 0..7 (rows past N read as zeros).
  float qf[32];
  {
    const int off = qi * (int)a.sq.s * 4 + 16 * hl;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rq, off + 32 * m, 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[4 * m + i] = x[i];
    }
  }

  f32x16 o[2];
  o[0] = zero16();
  o[1] = zero16();
  float m = -kInf, l = 0.f;
  const float c = a.scale_log2;

  auto kept = [&](int t) FA_INLINE -> bool {
    if (a.bmask == nullptr) return true;
    return a.bmask[(int64_t)(q0 / a.mask_block) * a.n_mask_k + (t * 64) / a.mask_block] != 0;
  };
  auto stage = [&](int t, float* kt, float* vt) FA_INLINE {
    stage_f32(rk, t * 64, ssk, kt, w, lane);
    stage_f32(rv, t * 64, ssv, vt, w, lane);
  };

  // Per-lane float offsets of the LDS reads: K row r, chunk 2 g + hl (g =
  // 0..7; key block kb adds 32 rows), and V column 32 db + r of the rows
  // 8 h + 4 hl + i (h = 0, 1, i = 0..3; further rows add multiples of 16,
  // which keep the swizzle).
  int kofs[8], vofs[16];
#pragma unroll
  for (int g = 0; g < 8; ++g) kofs[g] = foff(r, 8 * g + 4 * hl);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int db = 0; db < 2; ++db) vofs[8 * h + 2 * i + db] = foff(8 * h + 4 * hl + i, 32 * db + r);

  auto compute = [&](int t, const float* kt, const float* vt) FA_INLINE {
    const int k0 = t * 64;
    if (k0 > qw + 31 + (causal ? a.coff : a.Nk)) return;  // every key past this wave's queries
    // Fresh copies of the offsets for this tile: otherwise the compiler
    // keeps one register per buffer and offset live across the loop.
#pragma unroll
    for (int g = 0; g < 8; ++g) __asm__ volatile("" : "+v"(kofs[g]));
#pragma unroll
    for (int x = 0; x < 16; ++x) __asm__ volatile("" : "+v"(vofs[x]));
    // S^T of keys k0 + 32 kb + (0..31) x this wave's 32 queries.
    // Each K read (four steps) is issued one group ahead of its MFMAs;
    // scheduling fences keep the compiler from hoisting all of them.
    f32x16 s[2];
    s[0] = zero16();
    s[1] = zero16();
    auto kread = [&](int j) FA_INLINE {  // group j = 8 kb + g
      return *reinterpret_cast<const f32x4*>(kt + 2048 * (j >> 3) + kofs[j & 7]);
    };
    f32x4 kx = kread(0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const f32x4 cur = kx;
      if (j + 1 < 16) kx = kread(j + 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[j >> 3] = mfma_f32(cur[i], qf[4 * (j & 7) + i], s[j >> 3]);
      FA_FENCE();
    }
    // Element e of block kb holds key k0 + 32 kb + 8 (e / 4) + 4 hl + e % 4.
    const int lim = min(kv_len - 1, causal ? qi + a.coff : a.Nk) - k0 - 4 * hl;
    float mx = -kInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (32 * kb + 8 * (e >> 2) + (e & 3) > lim) s[kb][e] = -kInf;
        mx = fmaxf(mx, s[kb][e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx * c);
    const float m_use = (m_new == -kInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
    m = m_new;
    // Probabilities (dropped ones count in l but not in O).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        [[maybe_unused]] uint32_t word = 0;
        if constexpr (DROP) {
          uint32_t z[4] = {(uint32_t)((k0 + 32 * kb + 8 * g + 4 * hl) >> 2),
                           (uint32_t)(qi >> 2), (uint32_t)bh, a.drop.offset};
          philox_rounds(z, a.drop.seed_lo, a.drop.seed_hi, 0, 10);
          const int wi = qi & 3;
          word = wi == 0 ? z[0] : (wi == 1 ? z[1] : (wi == 2 ? z[2] : z[3]));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * g + i;
          const float p = fast_exp2(__builtin_fmaf(s[kb][e], c, -m_use));
          l += p;
          if constexpr (DROP)
            s[kb][e] = ((word >> (8 * i)) & 0xFFu) < a.drop.t ? p : 0.f;
          else
            s[kb][e] = p;
        }
      }
    }
    // O^T += V^T P^T over the 64 keys, four steps per group, the V reads of
    // a group issued one group ahead.
    // group j = 4 kb + e / 4: rows 32 kb + 8 (j % 4) + 4 hl + i, i.e. row
    // block 16 (2 kb + (j % 4) / 2) at offsets h = (j % 4) % 2
    auto vread = [&](int j, float (&dst)[8]) FA_INLINE {
      const int rb = 16 * (2 * (j >> 2) + ((j & 3) >> 1)), h = j & 1;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int db = 0; db < 2; ++db) dst[2 * i + db] = vt[64 * rb + vofs[8 * h + 2 * i + db]];
    };
    float vx[8], vc[8];
    vread(0, vx);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int x = 0; x < 8; ++x) vc[x] = vx[x];
      if (j + 1 < 8) vread(j + 1, vx);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int db = 0; db < 2; ++db)
          o[db] = mfma_f32(vc[2 * i + db], s[j >> 2][4 * (j & 3) + i], o[db]);
      FA_FENCE();
    }
  };

  int it = 0;
  while (it < ntk && !kept(it)) ++it;
  if (it < ntk) stage(it, s_k0, s_v0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Two tiles per trip so that each buffer is a fixed array.
  while (it < ntk) {
    int nx = it + 1;
    while (nx < ntk && !kept(nx)) ++nx;
    if (nx < ntk) stage(nx, s_k1, s_v1);
    compute(it, s_k0, s_v0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    it = nx;
    if (it >= ntk) break;
    nx = it + 1;
    while (nx < ntk && !kept(nx)) ++nx;
    if (nx < ntk) stage(nx, s_k0, s_v0);
    compute(it, s_k1, s_v1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    it = nx;
  }

  const float lt = l + __shfl_xor(l, 32, 64);
  if (qi < a.N) {
    float inv = lt > 0.f ? 1.f / lt : 0.f;
    if constexpr (DROP) inv *= a.drop.scale;
    float* op = (float*)a.o + b * a.so.b + hh * a.so.h + (int64_t)qi * a.so.s;
    // element e of block db holds O[qi][32 db + 8 (e / 4) + 4 hl + e % 4]
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = o[db][4 * j + i] * inv;
        *reinterpret_cast<f32x4*>(op + 32 * db + 8 * j + 4 * hl) = v4;
      }
    if (hl == 0)
      a.lse[(int64_t)bh * a.N + qi] = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -kInf;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, bool causal, hipStream_t stream) {
  FwdArgs copy = a;
  int cz = causal ? 1 : 0;
  void* args[] = {&copy, &cz};
  dim3 grid((unsigned)(((a.N + kBR - 1) / kBR) * a.B * a.H)), block(64 * kW);
  const void* fn = a.drop.t < 256 ? (const void*)&fwd_f32_kernel<true>
                                  : (const void*)&fwd_f32_kernel<false>;
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace fa
