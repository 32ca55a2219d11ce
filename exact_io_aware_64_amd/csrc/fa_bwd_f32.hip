// fp32 attention backward on the fp32 matrix cores (v_mfma_f32_32x32x2_f32).
//
// The backward pass keeps only the row statistic L of the forward and
// recomputes the probabilities tile by tile from it (researchpapers.dev
// explainer, "tiling and recomputation"; suanlizi.com summary,
// "recomputation"):
//   P = exp(s - L),  dP = dO V^T,  D_i = dot(dO_i, O_i),  dS = P (dP - D),
//   dV = P^T dO,     dK = scale dS^T Q,   dQ = scale dS K.
// Two kernels, as in the bf16 path's two roles, neither needing atomics:
//  * dq_f32_kernel, query-stationary: each wave owns 32 queries with their Q
//    and dO rows in registers; K/V tiles of 64 keys stream through LDS.
//    S^T = K Q^T and dP^T = V dO^T contract the head dimension (row reads of
//    the K and V tiles), dQ^T += K^T dS^T the keys (column reads of the K
//    tile, dS^T straight from the accumulator).  D comes from the lane's
//    dO and O rows.
//  * dkdv_f32_kernel, key-stationary: each wave owns 32 keys with their K and
//    V rows in registers; Q/dO tiles of 64 queries stream through LDS.
//    S = Q K^T and dP = dO V^T contract the head dimension, dV^T += dO^T P
//    and dK^T += Q^T dS the queries (column reads of the dO and Q tiles).
//    L and D of a tile's rows go to LDS next to the tile: D from the dO
//    rows in LDS and O rows fetched one tile ahead.
// Head dimension D = 32, 64 or 128.  The operand pairing and the LDS layout
// are those of fa_f32_tile.h; every
// product is fp32 accumulated in fp32, so results stay within ~1e-6 of
// exact.  Each 64-row tile is taken as two 32-row blocks so that only one
// block's S and dP accumulators are live at a time.
//
// Dropout with keep indicator Z and keep scale s: dV = (s Z P)^T dO,
// dP = s Z (dO V^T), dS = P (dP - D).  The keep bytes are those of the
// forward (Philox4x32-10, counter (j / 4, i / 4, b H + h, offset), pair (i, j)
// byte j % 4 of word i % 4).
#include "fa_f32_tile.h"

namespace fa {
namespace {

constexpr int kW = 4;         // waves per workgroup
constexpr int kBR = 32 * kW;  // query (dQ) or key (dK/dV) rows per workgroup

// The keep word of (query quad qq, key quad kq), word `wi` of the call.
__device__ __forceinline__ uint32_t keep_word(const Dropout& d, int kq, int qq, int bh, int wi) {
  uint32_t z[4] = {(uint32_t)kq, (uint32_t)qq, (uint32_t)bh, d.offset};
  philox_rounds(z, d.seed_lo, d.seed_hi, 0, 10);
  return wi == 0 ? z[0] : (wi == 1 ? z[1] : (wi == 2 ? z[2] : z[3]));
}

// ------------------------------------------------------------------- dQ

// Two waves per SIMD at D <= 64; at D = 128 the Q and dO rows alone take
// 128 registers and the four tiles 128 KiB of LDS: one wave per SIMD.
template <int D, bool DROP>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2, D == 128 ? 1 : 2))) void
dq_f32_kernel(BwdArgs a, int causal) {
  constexpr int kTileF = f32t::Geo<D>::kTileF;
  constexpr int NDB = D / 32;
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
      (const float*)a.q + b * a.sq.b + hh * a.sq.h, slice_bytes(a.N, a.sq.s, 4, D));
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(
      (const float*)a.dout + b * a.sdo.b + hh * a.sdo.h, slice_bytes(a.N, a.sdo.s, 4, D));
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(
      (const float*)a.o + b * a.so.b + hh * a.so.h, slice_bytes(a.N, a.so.s, 4, D));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(
      (const float*)a.k + b * a.sk.b + hh * a.sk.h, slice_bytes(a.Nk, a.sk.s, 4, D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(
      (const float*)a.v + b * a.sv.b + hh * a.sv.h, slice_bytes(a.Nk, a.sv.s, 4, D));
  const int ssk = (int)a.sk.s * 4, ssv = (int)a.sv.s * 4;

  // Q and dO fragments of this lane's query (rows past N read as zeros), D
  // from the dO and O rows (the two wave halves hold the two halves of them).
  float qf[D / 2], dof[D / 2];
  f32t::load_frag<D>(rq, qi, (int)a.sq.s * 4, hl, qf);
  f32t::load_frag<D>(rdo, qi, (int)a.sdo.s * 4, hl, dof);
  float Dq = 0.f;
  {
    float of_[D / 2];
    f32t::load_frag<D>(ro, qi, (int)a.so.s * 4, hl, of_);
#pragma unroll
    for (int x = 0; x < D / 2; ++x) Dq = __builtin_fmaf(dof[x], of_[x], Dq);
    Dq += __shfl_xor(Dq, 32, 64);
  }
  float L2 = kInf;  // +inf makes every probability of a dead or padding row 0
  if (qi < a.N) {
    const float L = a.lse[(int64_t)bh * a.N + qi];
    if (L != -kInf) L2 = L * kLog2e;
  }
  const float c = a.scale_log2;

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  auto kept = [&](int t) FA_INLINE -> bool {
    if (a.bmask == nullptr) return true;
    return a.bmask[(int64_t)(q0 / a.mask_block) * a.n_mask_k + (t * 64) / a.mask_block] != 0;
  };
  auto stage = [&](int t, float* kt, float* vt) FA_INLINE {
    f32t::stage<D, kW>(rk, t * 64, ssk, kt, w, lane);
    f32t::stage<D, kW>(rv, t * 64, ssv, vt, w, lane);
  };
  f32t::Offsets<D> of;
  of.init(r, hl);

  auto compute = [&](int t, const float* kt, const float* vt) FA_INLINE {
    const int k0 = t * 64;
    if (k0 > qw + 31 + (causal ? a.coff : a.Nk)) return;  // every key past this wave's queries
    of.refresh();
    // element e of block kb holds key k0 + 32 kb + 8 (e / 4) + 4 hl + e % 4
    const int lim = min(kv_len - 1, causal ? qi + a.coff : a.Nk) - k0 - 4 * hl;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 st = f32t::row_product<D>(kt, of, kb, qf);   // S^T
      f32x16 dpt = f32t::row_product<D>(vt, of, kb, dof);  // dP^T
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        [[maybe_unused]] uint32_t word = 0;
        if constexpr (DROP)
          word = keep_word(a.drop, (k0 + 32 * kb + 8 * g + 4 * hl) >> 2, qi >> 2, bh, qi & 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * g + i;
          const bool vis = 32 * kb + 8 * g + i <= lim;
          const float p = vis ? fast_exp2(__builtin_fmaf(st[e], c, -L2)) : 0.f;
          float dp = dpt[e];
          if constexpr (DROP)
            dp = ((word >> (8 * i)) & 0xFFu) < a.drop.t ? a.drop.scale * dp : 0.f;
          st[e] = p * (dp - Dq);  // dS^T
        }
      }
      f32t::col_product<D>(kt, of, kb, st, acc);  // dQ^T += K^T dS^T
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

  if (qi < a.N) {
    float* out = (float*)a.dq + b * a.sdq.b + hh * a.sdq.h + (int64_t)qi * a.sdq.s;
    f32t::store_rows<D>(out, hl, acc, a.scale);
  }
}

// ---------------------------------------------------------------- dK, dV

// One wave per SIMD at D >= 64: K and V rows, both accumulator sets, one
// block's S and dP and the O rows fetched for the next tile's D need more
// than the 256 registers of two waves.  Its work is almost all matrix
// instructions, whose dependent chains one wave keeps issuing back to back.
// At D = 32 everything fits in half of that: two waves per SIMD.
template <int D, bool DROP>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(D == 32 ? 2 : 1, D == 32 ? 2 : 1))) void
dkdv_f32_kernel(BwdArgs a, int causal) {
  constexpr int kTileF = f32t::Geo<D>::kTileF;
  constexpr int NDB = D / 32;
  constexpr int NQ = D / 16;  // 16-byte pieces of a quarter row
  __shared__ __attribute__((aligned(16))) float s_q0[kTileF];
  __shared__ __attribute__((aligned(16))) float s_g0[kTileF];
  __shared__ __attribute__((aligned(16))) float s_q1[kTileF];
  __shared__ __attribute__((aligned(16))) float s_g1[kTileF];
  __shared__ __attribute__((aligned(16))) float s_l2[2][64];  // L log2 e (+inf: no row)
  __shared__ __attribute__((aligned(16))) float s_d[2][64];   // D

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 31, hl = lane >> 5;
  const int BH = a.B * a.H;
  const int kt = (int)blockIdx.x / BH;  // key tile 0 sees the most queries (causal)
  const int bh = (int)blockIdx.x % BH;
  const int b = bh / a.H, hh = bh % a.H;
  const int k0 = kt * kBR, kw = k0 + 32 * w, kj = kw + r;

  int kv_len = a.Nk;
  if (a.seqlens) kv_len = min(max(a.seqlens[b], 0), a.Nk);

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(
      (const float*)a.q + b * a.sq.b + hh * a.sq.h, slice_bytes(a.N, a.sq.s, 4, D));
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(
      (const float*)a.dout + b * a.sdo.b + hh * a.sdo.h, slice_bytes(a.N, a.sdo.s, 4, D));
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(
      (const float*)a.o + b * a.so.b + hh * a.so.h, slice_bytes(a.N, a.so.s, 4, D));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(
      (const float*)a.k + b * a.sk.b + hh * a.sk.h, slice_bytes(a.Nk, a.sk.s, 4, D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(
      (const float*)a.v + b * a.sv.b + hh * a.sv.h, slice_bytes(a.Nk, a.sv.s, 4, D));
  const __amdgpu_buffer_rsrc_t rl =
      make_rsrc(a.lse + (int64_t)bh * a.N, (uint32_t)a.N * 4);
  const int ssq = (int)a.sq.s * 4, ssdo = (int)a.sdo.s * 4, sso = (int)a.so.s * 4;

  f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dkt[db] = dvt[db] = zero16();

  if (k0 < kv_len) {
    float kf[D / 2], vf[D / 2];
    f32t::load_frag<D>(rk, kj, (int)a.sk.s * 4, hl, kf);
    f32t::load_frag<D>(rv, kj, (int)a.sv.s * 4, hl, vf);
    const float c = a.scale_log2;
    const int nq = (a.N + 63) / 64;
    // causal: the first query that sees key k0 is k0 - coff
    const int qt_lo = causal ? max(0, k0 - a.coff) / 64 : 0;
    auto kept = [&](int t) FA_INLINE -> bool {
      if (a.bmask == nullptr) return true;
      return a.bmask[(int64_t)((t * 64) / a.mask_block) * a.n_mask_k + k0 / a.mask_block] != 0;
    };

    // Row statistics of a tile: thread (row, part) = (tid / 4, tid % 4)
    // takes a quarter of row `row`'s D = dot(dO, O): its O quarter is
    // fetched when the tile's copy is issued and its dO quarter read from
    // the tile once the copy has landed.
    const int srow = tid >> 2, spart = tid & 3;
    f32x4 oq[NQ];
    float lraw = 0.f;
    auto fetch_o = [&](int t) FA_INLINE {
      const int row = t * 64 + srow;
#pragma unroll
      for (int x = 0; x < NQ; ++x)
        oq[x] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, row * sso + D * spart + 16 * x, 0, 0));
      lraw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * row, 0, 0));
    };
    auto stage = [&](int t, float* qt_, float* gt_) FA_INLINE {
      f32t::stage<D, kW>(rq, t * 64, ssq, qt_, w, lane);
      f32t::stage<D, kW>(rdo, t * 64, ssdo, gt_, w, lane);
      fetch_o(t);
    };
    // After the tile's copy is visible to every wave: L and D of its rows.
    auto stats = [&](int t, const float* gt_, int buf) FA_INLINE {
      float dd = 0.f;
#pragma unroll
      for (int x = 0; x < NQ; ++x) {
        const f32x4 g4 =
            *reinterpret_cast<const f32x4*>(gt_ + f32t::foff<D>(srow, (D / 4) * spart + 4 * x));
#pragma unroll
        for (int i = 0; i < 4; ++i) dd = __builtin_fmaf(g4[i], oq[x][i], dd);
      }
      dd += quad_xor1(dd);
      dd += quad_xor2(dd);
      if (spart == 0) {
        const int row = t * 64 + srow;
        s_d[buf][srow] = dd;  // rows past N read as zeros: D = 0
        s_l2[buf][srow] = (row < a.N && lraw != -kInf) ? lraw * kLog2e : kInf;
      }
    };
    auto compute = [&](int t, const float* qt_, const float* gt_, int buf) FA_INLINE {
      const int qs = t * 64;
      // causal: no query of the tile sees any key of this wave
      if (causal && qs + 63 < kw - a.coff) return;
      // the offsets are recomputed per tile: registers are short here
      f32t::Offsets<D> of;
      of.init_here(lane);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        // S, then P as it enters dV (dropped pairs 0); dP, then dS.
        f32x16 sc = f32t::row_product<D>(qt_, of, qb, kf);
        f32x16 dp = f32t::row_product<D>(gt_, of, qb, vf);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // element e = 4 g + i holds query qs + 32 qb + 8 g + 4 hl + i
          const int qrow = 32 * qb + 8 * g + 4 * hl;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&s_l2[buf][qrow]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&s_d[buf][qrow]);
          [[maybe_unused]] uint32_t zw[4] = {0u, 0u, 0u, 0u};
          if constexpr (DROP) {
            zw[0] = (uint32_t)(kj >> 2);
            zw[1] = (uint32_t)((qs + qrow) >> 2);
            zw[2] = (uint32_t)bh;
            zw[3] = a.drop.offset;
            philox_rounds(zw, a.drop.seed_lo, a.drop.seed_hi, 0, 10);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * g + i;
            const int q = qs + qrow + i;
            const bool vis = kj < kv_len && (!causal || kj <= q + a.coff);
            const float p = vis ? fast_exp2(__builtin_fmaf(sc[e], c, -l4[i])) : 0.f;
            float dpe = dp[e], pe = p;
            if constexpr (DROP) {
              const bool keep = ((zw[i] >> (8 * (kj & 3))) & 0xFFu) < a.drop.t;
              dpe = keep ? a.drop.scale * dpe : 0.f;
              pe = keep ? p : 0.f;
            }
            sc[e] = pe;
            dp[e] = p * (dpe - d4[i]);
          }
        }
        f32t::col_product<D>(gt_, of, qb, sc, dvt);  // dV^T += dO^T P
        f32t::col_product<D>(qt_, of, qb, dp, dkt);  // dK^T += Q^T dS
      }
    };

    int it = qt_lo;
    while (it < nq && !kept(it)) ++it;
    if (it < nq) stage(it, s_q0, s_g0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it < nq) stats(it, s_g0, 0);
    __syncthreads();
    // Two tiles per trip so that each buffer is a fixed array.
    while (it < nq) {
      int nx = it + 1;
      while (nx < nq && !kept(nx)) ++nx;
      if (nx < nq) stage(nx, s_q1, s_g1);
      compute(it, s_q0, s_g0, 0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (nx < nq) stats(nx, s_g1, 1);
      __syncthreads();
      it = nx;
      if (it >= nq) break;
      nx = it + 1;
      while (nx < nq && !kept(nx)) ++nx;
      if (nx < nq) stage(nx, s_q0, s_g0);
      compute(it, s_q1, s_g1, 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (nx < nq) stats(nx, s_g0, 0);
      __syncthreads();
      it = nx;
    }
  }

  if (kj < a.Nk) {
    float* kout = (float*)a.dk + b * a.sdk.b + hh * a.sdk.h + (int64_t)kj * a.sdk.s;
    float* vout = (float*)a.dv + b * a.sdv.b + hh * a.sdv.h + (int64_t)kj * a.sdv.s;
    f32t::store_rows<D>(kout, hl, dkt, a.scale);
    f32t::store_rows<D>(vout, hl, dvt, DROP ? a.drop.scale : 1.f);
  }
}

template <int D>
hipError_t launch_bwd_f32_d(void** args, const BwdArgs& a, int phases, hipStream_t stream) {
  const dim3 block(64 * kW);
  const bool drop = a.drop.t < 256;
  if (phases & kPhaseDQ) {
    const dim3 grid((unsigned)(((a.N + kBR - 1) / kBR) * a.B * a.H));
    const void* fn =
        drop ? (const void*)&dq_f32_kernel<D, true> : (const void*)&dq_f32_kernel<D, false>;
    const hipError_t e = hipLaunchKernel(fn, grid, block, args, 0, stream);
    if (e != hipSuccess) return e;
  }
  if (phases & kPhaseDKDV) {
    const dim3 grid((unsigned)(((a.Nk + kBR - 1) / kBR) * a.B * a.H));
    const void* fn =
        drop ? (const void*)&dkdv_f32_kernel<D, true> : (const void*)&dkdv_f32_kernel<D, false>;
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a, bool causal, int phases, int d, hipStream_t stream) {
  BwdArgs copy = a;
  int cz = causal ? 1 : 0;
  void* args[] = {&copy, &cz};
  switch (d) {
    case 32: return launch_bwd_f32_d<32>(args, a, phases, stream);
    case 64: return launch_bwd_f32_d<64>(args, a, phases, stream);
    case 128: return launch_bwd_f32_d<128>(args, a, phases, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
