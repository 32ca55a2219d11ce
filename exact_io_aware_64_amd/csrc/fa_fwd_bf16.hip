// Fused attention forward for gfx950, bf16 inputs, fp32 accumulation.
//
// One workgroup (4 waves) owns 128 query rows of one (batch, head); each wave
// owns 32 of them and keeps its Q fragment in registers for the whole kernel.
// Key/value tiles of 64 rows stream through LDS (double-buffered: the global
// loads of tile t+1 are in flight while tile t is computed), so each K/V
// element is read from HBM/L2 once per workgroup and the N x N score matrix
// never leaves registers (suanlizi.com summary, "tiling" and "kernel fusion";
// researchpapers.dev explainer, "tiling and recomputation").
//
// The scores are computed transposed, S^T = K Q^T, on the 32x32x16 bf16 MFMA:
// in the accumulator layout each lane then holds 32 scores of a single query,
// so the row maximum and row sum need one exchange between the two wave
// halves instead of a reduction across 32 lanes.  The online softmax keeps a
// running maximum m (log2 units) and a running sum l per query and rescales
// the output accumulator when m grows (researchpapers.dev, "tiling and
// recomputation"; the max subtraction is the safe softmax of the llm-deploy
// note).  O^T = V^T P^T is accumulated on the same MFMA; the probabilities
// feed the B operand straight from the accumulator registers, and the V^T
// operand is read from the row-major V tile with LDS transpose reads.
//
// Tiles that the mask removes entirely are never loaded: causal and key
// padding shrink the key range, and a block mask is compacted into a list of
// kept tiles (suanlizi.com, "block-sparse attention").
#include "fa_device.h"

namespace fa {
namespace {

constexpr int kBR = 128;  // query rows per workgroup
// The running maximum is only moved (and O, l rescaled) when a tile's
// maximum exceeds it by more than this many log2 units; until then the
// probabilities are taken against the stale maximum and stay below
// 2^kSlack.  O = acc / l and L = m + log2(l) are unchanged by the choice of
// reference, so the result is the same up to rounding.
constexpr float kSlack = 8.f;

template <bool CAUSAL, bool SEQLEN, bool BMASK>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kTile * kRowStride];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[2][kTile * kRowStride];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 31, hl = lane >> 5;
  const int BH = a.B * a.H;
  const int nqt = (a.N + kBR - 1) / kBR;
  const int id = blockIdx.x;
  // Causal: the longest query tiles are dispatched first.  Consecutive ids
  // walk the heads, so with B*H a multiple of 8 all tiles of one head land
  // on the same XCD and share its L2.
  const int qt = CAUSAL ? (nqt - 1 - id / BH) : (id / BH);
  const int bh = id % BH;
  const int b = bh / a.H, hh = bh % a.H;
  const int q0 = qt * kBR;
  const int qw = q0 + 32 * w;  // first query of this wave
  const int qi = qw + r;       // this lane's query

  int kv_len = a.N;
  if constexpr (SEQLEN) kv_len = min(max(a.seqlens[b], 0), a.N);
  int kend = kv_len;
  if constexpr (CAUSAL) kend = min(kend, q0 + kBR);
  const int ntk = (kend + kTile - 1) / kTile;

  int nlist = ntk;
  [[maybe_unused]] uint16_t* tlist = nullptr;
  if constexpr (BMASK) {
    __shared__ uint16_t s_list[kMaxListTiles];
    __shared__ int s_scan[4];
    tlist = s_list;
    const int row = q0 / a.mask_block;
    nlist = build_tile_list(s_list, s_scan, a.bmask + (int64_t)row * a.n_mask_tiles, 1,
                            a.n_mask_tiles, a.mask_block / kTile, 0, ntk);
  }

  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc((const uint16_t*)a.q + b * a.sq.b + hh * a.sq.h, slice_bytes(a.N, a.sq.s, 2));
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc((const uint16_t*)a.k + b * a.sk.b + hh * a.sk.h, slice_bytes(a.N, a.sk.s, 2));
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc((const uint16_t*)a.v + b * a.sv.b + hh * a.sv.h, slice_bytes(a.N, a.sv.s, 2));
  const int ssk = (int)a.sk.s * 2, ssv = (int)a.sv.s * 2;

  // Q fragment: B operand of S^T = K Q^T, lane (r, hl) holds
  // Q[qi][16 ks + 8 hl .. +7].  Rows past N read as zeros.
  bf16x8 qf[4];
  {
    const int off = qi * (int)a.sq.s * 2 + 16 * hl;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(ldb16(rq, off + 32 * ks));
  }

  f32x16 o[2] = {zero16(), zero16()};
  float m = -kInf, l = 0.f;
  const float c = a.scale_log2;

  // Staging roles: rows tid/8 and tid/8 + 32 of the K and V tiles, 16-byte
  // column tid%8, stored row-major.
  const int sr = tid >> 3, sc = tid & 7;
  const int k_off0 = sr * ssk + 16 * sc, k_off1 = (sr + 32) * ssk + 16 * sc;
  const int v_off0 = sr * ssv + 16 * sc, v_off1 = (sr + 32) * ssv + 16 * sc;
  const int trl = tr_lane_offset(lane);
  uint4 kreg[2], vreg[2];
  auto tile_at = [&](int it) -> int {
    if constexpr (BMASK) return tlist[it];
    return it;
  };
  auto gload = [&](int t) {
    const int k0 = t * kTile;
    kreg[0] = ldb16(rk, k_off0 + k0 * ssk);
    kreg[1] = ldb16(rk, k_off1 + k0 * ssk);
    vreg[0] = ldb16(rv, v_off0 + k0 * ssv);
    vreg[1] = ldb16(rv, v_off1 + k0 * ssv);
  };
  auto swrite = [&](int buf) {
    store_row16(s_k[buf], sr, sc, kreg[0]);
    store_row16(s_k[buf], sr + 32, sc, kreg[1]);
    store_row16(s_v[buf], sr, sc, vreg[0]);
    store_row16(s_v[buf], sr + 32, sc, vreg[1]);
  };

  if (nlist > 0) {
    gload(tile_at(0));
    swrite(0);
  }
  __syncthreads();

  for (int it = 0; it < nlist; ++it) {
    const int buf = it & 1;
    const int k0 = tile_at(it) * kTile;
    if (it + 1 < nlist) gload(tile_at(it + 1));

    const bool active = !CAUSAL || (k0 <= qw + 31);
    if (active) {
      const uint16_t* ks_ = s_k[buf];
      const uint16_t* vs_ = s_v[buf];
      // S^T for keys k0 .. k0+63 as two interleaved 32-key accumulator chains.
      bf16x8 ka[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          ka[kb][ks] = lds_row8(ks_ + (32 * kb + r) * kRowStride + 16 * ks + 8 * hl);
      f32x16 s[2] = {zero16(), zero16()};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s[0] = mfma32(ka[0][ks], qf[ks], s[0]);
        s[1] = mfma32(ka[1][ks], qf[ks], s[1]);
      }
      const bool need_mask = (k0 + kTile > kv_len) || (CAUSAL && k0 + kTile - 1 > qw);
      if (need_mask) {
        // element e of block kb holds key k0 + 4*hl + off(kb, e); it is
        // visible iff off <= lim
        const int last = CAUSAL ? min(kv_len - 1, qi) : kv_len - 1;
        const int lim = last - k0 - 4 * hl;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * kb + 8 * (e >> 2) + (e & 3) > lim) s[kb][e] = -kInf;
      }
      float mx = -kInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
      const float mt = half_max(mx) * c;  // tile maximum, log2 units
      const bool grow = mt > m + kSlack;
      if (__any(grow)) {
        // alpha is 0 when m was -inf (nothing accumulated yet) and exactly 1
        // in lanes that keep their reference.
        const float alpha = grow ? fast_exp2(m - mt) : 1.f;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
        m = grow ? mt : m;
      }
      const float m_use = (m == -kInf) ? 0.f : m;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][e], c, -m_use));
          s[kb][e] = p;
          rs += p;
        }
      l += rs;
      // O^T[d][q] += sum_key V[key][d] P[q][key]; contraction slot e of step
      // st maps to key 16*st + 4*hl + e (e < 4) or 16*st + 8 + 4*hl + e - 4.
      bf16x8 va[4][2];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int db = 0; db < 2; ++db)
          va[st][db] = tr_operand(vs_ + trl + 16 * st * kRowStride + 32 * db);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 pb = pack8(s[st >> 1], 8 * (st & 1));
        o[0] = mfma32(va[st][0], pb, o[0]);
        o[1] = mfma32(va[st][1], pb, o[1]);
      }
    }
    if (it + 1 < nlist) swrite(buf ^ 1);
    __syncthreads();
  }

  const float lt = half_sum(l);
  if (qi < a.N) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* op = (uint16_t*)a.o + b * a.so.b + hh * a.so.h + (int64_t)qi * a.so.s;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = (__bf16)(o[db][4 * j + i] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * j + 4 * hl) = v4;
      }
    if (hl == 0)
      a.lse[(int64_t)bh * a.N + qi] =
          lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -kInf;
  }
}

template <bool C, bool S, bool M>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.N + kBR - 1) / kBR;
  dim3 grid((unsigned)(nqt * a.B * a.H)), block(256);
  FwdArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel((const void*)&fwd_bf16_kernel<C, S, M>, grid, block, args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, bool causal, hipStream_t stream) {
  const bool s = a.seqlens != nullptr, m = a.bmask != nullptr;
  if (causal) {
    if (s) return m ? launch<true, true, true>(a, stream) : launch<true, true, false>(a, stream);
    return m ? launch<true, false, true>(a, stream) : launch<true, false, false>(a, stream);
  }
  if (s) return m ? launch<false, true, true>(a, stream) : launch<false, true, false>(a, stream);
  return m ? launch<false, false, true>(a, stream) : launch<false, false, false>(a, stream);
}

}  // namespace fa
