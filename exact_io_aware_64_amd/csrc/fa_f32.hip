// fp32 attention backward on the vector ALUs (the fp32 forward runs on the
// matrix cores, fa_fwd_f32.hip).
//
// Same tiled algorithm as the bf16 kernels -- K/V (or Q/dO) tiles of 64 rows
// staged in LDS, probabilities recomputed from L (researchpapers.dev
// explainer, "tiling and recomputation") -- but every product is an fp32
// FMA, so results stay within ~1e-6 of exact.  One thread owns one query
// (dQ) or one key (dK/dV); every thread of a workgroup reads the same LDS
// row at the same time (a broadcast).  This path serves full-precision
// callers and small problems; the bf16 MFMA kernels are the throughput path.
// With dropout, each thread makes one Philox call per four consecutive pairs
// of its loop: the block of query i and keys j..j+3 gives key j % 4's byte
// of word i % 4 (dQ); the block of queries i..i+3 and key j gives byte j % 4
// of each word (dK/dV).
#include "fa_device.h"

namespace fa {
namespace {

constexpr int kD = 64;

__device__ __forceinline__ bool tile_kept(const uint8_t* bmask, int n_mask_k, int mask_block,
                                          int qrow, int kcol) {
  return bmask == nullptr ||
         bmask[(int64_t)(qrow / mask_block) * n_mask_k + kcol / mask_block] != 0;
}

__device__ __forceinline__ void load_row(float* dst, const float* src) {
#pragma unroll
  for (int e = 0; e < kD; e += 4) {
    const float4 x = *reinterpret_cast<const float4*>(src + e);
    dst[e] = x.x;
    dst[e + 1] = x.y;
    dst[e + 2] = x.z;
    dst[e + 3] = x.w;
  }
}

__device__ __forceinline__ void store_row(float* dst, const float* src, float mul) {
#pragma unroll
  for (int e = 0; e < kD; e += 4)
    *reinterpret_cast<float4*>(dst + e) =
        make_float4(src[e] * mul, src[e + 1] * mul, src[e + 2] * mul, src[e + 3] * mul);
}

__device__ __forceinline__ void stage_row(float* lds_row, const float* g, bool in) {
#pragma unroll
  for (int e = 0; e < kD; e += 4)
    *reinterpret_cast<float4*>(lds_row + e) =
        in ? *reinterpret_cast<const float4*>(g + e) : make_float4(0.f, 0.f, 0.f, 0.f);
}

__device__ __forceinline__ float dot_lds(const float* x, const float* lds_row) {
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < kD; ++e) acc = __builtin_fmaf(x[e], lds_row[e], acc);
  return acc;
}

// The Philox call of pairs (queries 4 qq .. +3, keys 4 kq .. +3) of slice bh.
__device__ __forceinline__ void drop_call(uint32_t (&w)[4], const Dropout& d, int qq, int kq,
                                          int bh) {
  w[0] = (uint32_t)kq;
  w[1] = (uint32_t)qq;
  w[2] = (uint32_t)bh;
  w[3] = d.offset;
  philox_rounds(w, d.seed_lo, d.seed_hi, 0, 10);
}

__device__ __forceinline__ bool keep_byte(uint32_t word, int byte, uint32_t t) {
  return ((word >> (8 * byte)) & 0xFFu) < t;
}

// w[i] for a run-time i, by selects (an indexed private array would live in
// scratch memory).
__device__ __forceinline__ uint32_t pick4(const uint32_t (&w)[4], int i) {
  const uint32_t lo = (i & 1) ? w[1] : w[0], hi = (i & 1) ? w[3] : w[2];
  return (i & 2) ? hi : lo;
}

// dQ for one query per thread.
template <bool DROP>
__global__ __launch_bounds__(64) void dq_f32_kernel(BwdArgs a, int causal) {
  __shared__ __attribute__((aligned(16))) float s_k[kTile * kD];
  __shared__ __attribute__((aligned(16))) float s_v[kTile * kD];
  const int tid = threadIdx.x;
  const int BH = a.B * a.H;
  const int qt = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int b = bh / a.H, hh = bh % a.H;
  const int q0 = qt * kTile, qi = q0 + tid;
  int kv_len = a.Nk;
  if (a.seqlens) kv_len = min(max(a.seqlens[b], 0), a.Nk);
  const int kend = causal ? min(kv_len, q0 + kTile + a.coff) : kv_len;
  const float* K = (const float*)a.k + b * a.sk.b + hh * a.sk.h;
  const float* V = (const float*)a.v + b * a.sv.b + hh * a.sv.h;

  float q[kD], g[kD], acc[kD];
  float D = 0.f, L2 = kInf;
  if (qi < a.N) {
    load_row(q, (const float*)a.q + b * a.sq.b + hh * a.sq.h + (int64_t)qi * a.sq.s);
    load_row(g, (const float*)a.dout + b * a.sdo.b + hh * a.sdo.h + (int64_t)qi * a.sdo.s);
    load_row(acc, (const float*)a.o + b * a.so.b + hh * a.so.h + (int64_t)qi * a.so.s);
#pragma unroll
    for (int e = 0; e < kD; ++e) D = __builtin_fmaf(g[e], acc[e], D);
    const float L = a.lse[(int64_t)bh * a.N + qi];
    if (L != -kInf) L2 = L * kLog2e;
  } else {
    for (int e = 0; e < kD; ++e) q[e] = g[e] = 0.f;
  }
  for (int e = 0; e < kD; ++e) acc[e] = 0.f;
  const float c = a.scale_log2;

  for (int k0 = 0; k0 < kend; k0 += kTile) {
    if (!tile_kept(a.bmask, a.n_mask_k, a.mask_block, q0, k0)) continue;
    const int kk = k0 + tid;
    stage_row(s_k + tid * kD, K + (int64_t)kk * a.sk.s, kk < a.Nk);
    stage_row(s_v + tid * kD, V + (int64_t)kk * a.sv.s, kk < a.Nk);
    __syncthreads();
    [[maybe_unused]] uint32_t zw[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < kTile; ++j) {
      const int key = k0 + j;
      const bool vis = key < kv_len && (!causal || key <= qi + a.coff);
      const float s = dot_lds(q, s_k + j * kD);
      const float p = vis ? fast_exp2(__builtin_fmaf(s, c, -L2)) : 0.f;
      float dp = dot_lds(g, s_v + j * kD);
      if constexpr (DROP) {
        if ((j & 3) == 0) drop_call(zw, a.drop, qi >> 2, key >> 2, bh);
        dp = keep_byte(pick4(zw, qi & 3), j & 3, a.drop.t) ? a.drop.scale * dp : 0.f;
      }
      const float ds = p * (dp - D);
#pragma unroll
      for (int e = 0; e < kD; ++e) acc[e] = __builtin_fmaf(ds, s_k[j * kD + e], acc[e]);
    }
    __syncthreads();
  }
  if (qi < a.N)
    store_row((float*)a.dq + b * a.sdq.b + hh * a.sdq.h + (int64_t)qi * a.sdq.s, acc, a.scale);
}

// dK, dV for one key per thread.  Each staged query row also gets its
// D_i = dot(dO_i, O_i), computed by the thread that stages it.
template <bool DROP>
__global__ __launch_bounds__(64) void dkdv_f32_kernel(BwdArgs a, int causal) {
  __shared__ __attribute__((aligned(16))) float s_q[kTile * kD];
  __shared__ __attribute__((aligned(16))) float s_g[kTile * kD];
  __shared__ float s_l2[kTile], s_d[kTile];
  const int tid = threadIdx.x;
  const int BH = a.B * a.H;
  const int kt = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int b = bh / a.H, hh = bh % a.H;
  const int k0 = kt * kTile, kj = k0 + tid;
  int kv_len = a.Nk;
  if (a.seqlens) kv_len = min(max(a.seqlens[b], 0), a.Nk);
  const float* Q = (const float*)a.q + b * a.sq.b + hh * a.sq.h;
  const float* G = (const float*)a.dout + b * a.sdo.b + hh * a.sdo.h;
  const float* O = (const float*)a.o + b * a.so.b + hh * a.so.h;

  float kr[kD], vr[kD], dk[kD], dv[kD];
  if (kj < a.Nk) {
    load_row(kr, (const float*)a.k + b * a.sk.b + hh * a.sk.h + (int64_t)kj * a.sk.s);
    load_row(vr, (const float*)a.v + b * a.sv.b + hh * a.sv.h + (int64_t)kj * a.sv.s);
  } else {
    for (int e = 0; e < kD; ++e) kr[e] = vr[e] = 0.f;
  }
  for (int e = 0; e < kD; ++e) dk[e] = dv[e] = 0.f;
  const float c = a.scale_log2;

  if (k0 < kv_len) {
    // causal: the first query that sees key k0 is k0 - coff
    for (int qs = causal ? max(0, k0 - a.coff) / kTile * kTile : 0; qs < a.N; qs += kTile) {
      if (!tile_kept(a.bmask, a.n_mask_k, a.mask_block, qs, k0)) continue;
      const int qq = qs + tid;
      stage_row(s_q + tid * kD, Q + (int64_t)qq * a.sq.s, qq < a.N);
      stage_row(s_g + tid * kD, G + (int64_t)qq * a.sdo.s, qq < a.N);
      const float L = qq < a.N ? a.lse[(int64_t)bh * a.N + qq] : -kInf;
      s_l2[tid] = (L == -kInf) ? kInf : L * kLog2e;
      float dd = 0.f;
      if (qq < a.N) {
        const float* orow = O + (int64_t)qq * a.so.s;
        const float* grow = G + (int64_t)qq * a.sdo.s;
        for (int e = 0; e < kD; ++e) dd = __builtin_fmaf(grow[e], orow[e], dd);
      }
      s_d[tid] = dd;
      __syncthreads();
      [[maybe_unused]] uint32_t zw[4] = {0u, 0u, 0u, 0u};
      for (int i = 0; i < kTile; ++i) {
        const int q = qs + i;
        const bool vis = kj < kv_len && (!causal || kj <= q + a.coff);
        const float s = dot_lds(kr, s_q + i * kD);
        float p = vis ? fast_exp2(__builtin_fmaf(s, c, -s_l2[i])) : 0.f;
        float dp = dot_lds(vr, s_g + i * kD);
        float pv = p;  // the weight of dO_i in dV
        if constexpr (DROP) {
          if ((i & 3) == 0) drop_call(zw, a.drop, q >> 2, kj >> 2, bh);
          const bool keep = keep_byte(pick4(zw, i & 3), kj & 3, a.drop.t);
          dp = keep ? a.drop.scale * dp : 0.f;
          pv = keep ? p : 0.f;
        }
        const float ds = p * (dp - s_d[i]);
#pragma unroll
        for (int e = 0; e < kD; ++e) {
          dv[e] = __builtin_fmaf(pv, s_g[i * kD + e], dv[e]);
          dk[e] = __builtin_fmaf(ds, s_q[i * kD + e], dk[e]);
        }
      }
      __syncthreads();
    }
  }
  if (kj < a.Nk) {
    store_row((float*)a.dk + b * a.sdk.b + hh * a.sdk.h + (int64_t)kj * a.sdk.s, dk, a.scale);
    store_row((float*)a.dv + b * a.sdv.b + hh * a.sdv.h + (int64_t)kj * a.sdv.s, dv,
              DROP ? a.drop.scale : 1.f);
  }
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a, bool causal, int phases, hipStream_t stream) {
  BwdArgs copy = a;
  int cz = causal ? 1 : 0;
  void* args[] = {&copy, &cz};
  const dim3 block(64);
  const bool drop = a.drop.t < 256;
  if (phases & kPhaseDQ) {
    const dim3 grid((unsigned)(((a.N + kTile - 1) / kTile) * a.B * a.H));
    const void* fn = drop ? (const void*)&dq_f32_kernel<true> : (const void*)&dq_f32_kernel<false>;
    hipError_t e = hipLaunchKernel(fn, grid, block, args, 0, stream);
    if (e != hipSuccess) return e;
  }
  if (phases & kPhaseDKDV) {
    const dim3 grid((unsigned)(((a.Nk + kTile - 1) / kTile) * a.B * a.H));
    const void* fn =
        drop ? (const void*)&dkdv_f32_kernel<true> : (const void*)&dkdv_f32_kernel<false>;
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
  }
  return hipSuccess;
}

}  // namespace fa
