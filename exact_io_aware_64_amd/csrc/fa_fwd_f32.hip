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
// owns 32 of them, with its Q rows in registers.  Head dimension D = 32, 64
// or 128; at D = 128 the four double-buffered tiles fill 128 KiB of LDS, so
// one workgroup (one wave per SIMD) runs per CU.  S^T = K Q^T contracts the
// head dimension (row reads of the K tile), O^T += V^T P^T the keys (column
// reads of the V tile, the probabilities straight from the S^T accumulator);
// the operand pairing and the LDS layout are those of fa_f32_tile.h.  The
// accumulators hold S^T and O^T with one query per lane column: the softmax
// needs no transposition and O rows leave as 16-byte stores.  Tiles are
// copied straight from memory into LDS, double-buffered.
//
// Masks as in the bf16 forward: key j is visible to query i iff j < the
// sequence's key length and (without the causal mask, or) j <= i + N_k - N,
// and a block mask drops whole 128 x 128 tiles before they are loaded.
// Dropout uses the same Philox4x32-10 keep bytes as the other kernels: the
// call with counter (j / 4, i / 4, b H + h, offset) gives pair (i, j) byte
// j % 4 of word i % 4.
#include "fa_f32_tile.h"

namespace fa {
namespace {

constexpr int kW = 4;         // waves per workgroup
constexpr int kBR = 32 * kW;  // query rows per workgroup

// Two waves per SIMD at D <= 64 (the LDS holds two workgroups'
// double-buffered tiles), one at D = 128.
template <int D, bool DROP>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2, D == 128 ? 1 : 2))) void
fwd_f32_kernel(FwdArgs a, int causal) {
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
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(
      (const float*)a.k + b * a.sk.b + hh * a.sk.h, slice_bytes(a.Nk, a.sk.s, 4, D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(
      (const float*)a.v + b * a.sv.b + hh * a.sv.h, slice_bytes(a.Nk, a.sv.s, 4, D));
  const int ssk = (int)a.sk.s * 4, ssv = (int)a.sv.s * 4;

  // Q[qi][8 g + 4 hl .. +3] for g < D / 8 (rows past N read as zeros).
  float qf[D / 2];
  f32t::load_frag<D>(rq, qi, (int)a.sq.s * 4, hl, qf);

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = zero16();
  float m = -kInf, l = 0.f;
  const float c = a.scale_log2;

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
    // S^T of keys k0 + 32 kb + (0..31) x this wave's 32 queries.
    f32x16 s[2];
    s[0] = f32t::row_product<D>(kt, of, 0, qf);
    s[1] = f32t::row_product<D>(kt, of, 1, qf);
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
    for (int db = 0; db < NDB; ++db)
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
    // O^T += V^T P^T over the 64 keys.
    f32t::col_product<D>(vt, of, 0, s[0], o);
    f32t::col_product<D>(vt, of, 1, s[1], o);
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
    f32t::store_rows<D>(op, hl, o, inv);
    if (hl == 0)
      a.lse[(int64_t)bh * a.N + qi] = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -kInf;
  }
}

template <int D>
const void* fwd_f32_fn(bool drop) {
  return drop ? (const void*)&fwd_f32_kernel<D, true> : (const void*)&fwd_f32_kernel<D, false>;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, bool causal, int d, hipStream_t stream) {
  FwdArgs copy = a;
  int cz = causal ? 1 : 0;
  void* args[] = {&copy, &cz};
  dim3 grid((unsigned)(((a.N + kBR - 1) / kBR) * a.B * a.H)), block(64 * kW);
  const bool drop = a.drop.t < 256;
  const void* fn = d == 32    ? fwd_f32_fn<32>(drop)
                   : d == 64  ? fwd_f32_fn<64>(drop)
                   : d == 128 ? fwd_f32_fn<128>(drop)
                              : nullptr;
  if (fn == nullptr) return hipErrorInvalidValue;
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace fa
