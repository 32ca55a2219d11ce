// Attention backward for gfx950, bf16 inputs, fp32 accumulation.
//
// The pages only say that the backward pass keeps the softmax statistics and
// recomputes the attention blocks from them instead of reading a stored
// N x N matrix (researchpapers.dev explainer, "tiling and recomputation";
// suanlizi.com summary, "recomputation").  With f = sum(dO * O) the
// gradients are
//   P = exp(s - L),  dP = dO V^T,  D_i = dot(dO_i, O_i),  dS = P * (dP - D),
//   dV = P^T dO,     dK = scale dS^T Q,   dQ = scale dS K.
//
// One kernel, launched once, whose workgroups take one of two roles; no
// gradient needs atomics or a transpose of dS, and the roles share nothing:
//  * dQ role: query-stationary, like the forward.  Each lane owns one query
//    with its Q, dO fragments, L and D in registers; K/V tiles stream through
//    LDS.  S^T = K Q^T and
//    dP^T = V dO^T come out of the MFMA with one query per lane, and
//    dQ^T = K^T dS^T takes dS^T straight from the accumulator.
//  * dK/dV role: key-stationary.  Each lane owns one key with its K, V
//    fragments in registers; Q and dO tiles, L and D stream through LDS.  S = Q K^T and dP = dO V^T
//    come out with one key per lane, which is exactly the B operand of
//    dV^T = dO^T P and dK^T = Q^T dS.
// One launch carries both roles, heaviest work first, so that the GPU stays
// busy to the end without a second kernel's launch gap and tail.  It is
// preceded by a small pass that writes D_i = dot(dO_i, O_i) of every query
// row to the workspace: the dK/dV role would otherwise copy an O tile into
// LDS next to every Q and dO tile it stages, only to form D (a third more
// tile traffic and LDS writes; the pass measured 4-6 % faster at 16K causal
// and 64K block-sparse, and even at 1K).  Masked
// tiles are skipped exactly as in the forward pass.
//
// Dropout (DROP), with keep indicator Z and keep scale s:
//   dV = (s Z P)^T dO,  dP = s Z (dO V^T),  dS = P (dP - D),  D_i = dot(dO_i, O_i).
// Each role regenerates the forward pass's keep bytes, one Philox call per
// lane and 32 x 32 block, in its MFMA-only slots; the dK/dV role holds the
// pairs key-major and transposes the bytes of its call first.  There dP no
// longer starts at -D (a dropped pair still needs -P D), so -D is read from
// LDS next to the pair instead.
#pragma once

#include <type_traits>

#include "fa_device.h"

namespace fa {
namespace {

constexpr int kBQ = 128;   // dQ role: query rows per workgroup
constexpr int kBK = 128;   // dK/dV role: key rows per workgroup

// Issues, at slot t, the chunks c (0..7) of a half tile that are spread over
// the nw slots starting at t0, chunk c in slot t0 + c nw / 8: the chunks with
// c nw / 8 == t - t0 (8 / nw of them when nw < 8, else at most one).
template <int T0, int NW, class F>
__device__ __forceinline__ void spread_chunks(int t, F&& f) {
  const int u = t - T0;
  if (u < 0 || u >= NW) return;
  const int c_lo = (8 * u + NW - 1) / NW, c_hi = (8 * (u + 1) + NW - 1) / NW;
#pragma unroll
  for (int cc = 0; cc < (8 + NW - 1) / NW; ++cc)
    if (c_lo + cc < c_hi && c_lo + cc < 8) f(c_lo + cc);
}

// ------------------------------------------------------------------ dQ (+D)

// dQ for the 128 queries of work item `item` (query tile, batch, head).
// s_k0/s_v0 and s_k1/s_v1 are the two K/V tile buffers.
template <int D, bool CAUSAL, bool SEQLEN, bool BMASK, bool DROP>
__device__ __forceinline__ void dq_role(const BwdArgs& a, int item, uint16_t* s_k0,
                                        uint16_t* s_v0, uint16_t* s_k1, uint16_t* s_v1,
                                        uint16_t* s_list, int* s_scan) {
  constexpr int KS = D / 16;  // contraction steps over d
  constexpr int DB = D / 32;  // 32-row blocks of dQ^T
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = tid >> 6;
  const int r = lane & 31, hl = lane >> 5;
  const int BH = a.B * a.H;
  const int nqt = (a.N + kBQ - 1) / kBQ;
  const int qt = CAUSAL ? (nqt - 1 - item / BH) : (item / BH);
  const int bh = item % BH;
  const int b = bh / a.H, hh = bh % a.H;
  const int q0 = qt * kBQ;
  const int qw = q0 + 32 * w;
  const int qi = qw + r;

  int kv_len = a.Nk;
  if constexpr (SEQLEN) kv_len = min(max(a.seqlens[b], 0), a.Nk);
  int kend = kv_len;
  if constexpr (CAUSAL) kend = max(0, min(kend, q0 + kBQ + a.coff));
  const int ntk = (kend + kTile - 1) / kTile;

  int nlist = ntk;
  [[maybe_unused]] uint16_t* tlist = nullptr;
  if constexpr (BMASK) {
    tlist = s_list;
    const int row = q0 / a.mask_block;
    nlist = build_tile_list(s_list, s_scan, a.bmask + (int64_t)row * a.n_mask_k, 1,
                            a.n_mask_k, a.mask_block / kTile, 0, ntk);
  }

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(
      (const uint16_t*)a.q + b * a.sq.b + hh * a.sq.h, slice_bytes(a.N, a.sq.s, 2, D));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(
      (const uint16_t*)a.k + b * a.sk.b + hh * a.sk.h, slice_bytes(a.Nk, a.sk.s, 2, D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(
      (const uint16_t*)a.v + b * a.sv.b + hh * a.sv.h, slice_bytes(a.Nk, a.sv.s, 2, D));
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(
      (const uint16_t*)a.dout + b * a.sdo.b + hh * a.sdo.h, slice_bytes(a.N, a.sdo.s, 2, D));
  const int ssk = (int)a.sk.s * 2, ssv = (int)a.sv.s * 2;

  // Q and dO fragments (B operands, lane (r, hl) holds row qi, columns
  // 16 ks + 8 hl .. +7) and D_i from the pre-pass.
  bf16x8 qf[KS], dof[KS];
  float Dq = 0.f;
  {
    const int oq = qi * (int)a.sq.s * 2 + 16 * hl;
    const int odo = qi * (int)a.sdo.s * 2 + 16 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = as_bf16x8(ldb16(rq, oq + 32 * ks));
      dof[ks] = as_bf16x8(ldb16(rdo, odo + 32 * ks));
    }
    if (qi < a.N) Dq = a.dsum[(int64_t)bh * a.N + qi];
  }
  float L2 = kInf;  // +inf makes every probability of a dead or padding row 0
  if (qi < a.N) {
    const float L = a.lse[(int64_t)bh * a.N + qi];
    if (L != -kInf) L2 = L * kLog2e;
  }
  const float c = a.scale_log2;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero16();

  // Per-lane LDS offsets: K and V rows (A operands of S^T and dP^T) and K^T
  // transpose reads (A operand of dQ^T).
  int roff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) roff[ks] = row_off(r, hl, ks);
  int troff[2][2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int db = 0; db < 2; ++db) troff[hi][db] = tr_off(lane, hi, db);

  auto tile_at = [&](int it) FA_INLINE -> int {
    if constexpr (BMASK) return tlist[it];
    return it;
  };
  auto stage = [&](int t, uint16_t* kt, uint16_t* vt) FA_INLINE {
#pragma unroll
    for (int j = 0; j < (D > 64 ? D / 64 : 1); ++j) {
      stage_tile(rk, t * kTile, ssk, kt + j * kTileElems, w, lane, 128 * j);
      stage_tile(rv, t * kTile, ssv, vt + j * kTileElems, w, lane, 128 * j);
    }
  };

  // One 64-key tile as 6 KS MFMA issue slots separated by scheduling fences
  // (for D = 64:
  //   slots  0.. 7  S^T, dP^T of keys  0..31                 (MFMA)
  //   slots  8..15  S^T, dP^T of keys 32..63                 (MFMA) | P, dS of keys 0..31
  //   slots 16..23  dQ^T += K^T dS^T (steps 0..3)            (MFMA) | P, dS of keys 32..63)
  // with each LDS operand read four slots ahead.  dS of keys 32..47 is done
  // by slot 19 and of 48..63 by slot 21, ahead of the steps that use them.
  // Other D: 4 KS slots of S^T and dP^T, then 4 DB of dQ^T, the dS chunks of
  // each half spread evenly over the slots that follow the half.
  auto body = [&](auto mask_c, const uint16_t* kt, const uint16_t* vt, int k0) FA_INLINE {
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr int kLead = 4;
    constexpr int NS = 6 * KS;
    // Without dropout dP^T starts at -D, so the MFMAs leave dP - D.
    f32x16 st[2] = {zero16(), zero16()}, dpt[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) dpt[kb][e] = DROP ? 0.f : -Dq;
    uint32_t pkd[4][4];  // bf16 pairs of dS per step
    bf16x8 opa[NS];
    [[maybe_unused]] DropBlock zb[2];  // keep bytes of the two halves
    [[maybe_unused]] int lim = 0;
    if constexpr (MASK) lim = (CAUSAL ? min(kv_len - 1, qi + a.coff) : kv_len - 1) - k0 - 4 * hl;
    // A operand of slot t
    auto load_a = [&](int t) FA_INLINE {
      if (t < 4 * KS) {
        const int kb = t / (2 * KS), ks = (t % (2 * KS)) >> 1;
        opa[t] = tile_row8(((t & 1) ? vt : kt) + (ks >> 2) * kTileElems,
                           2048 * kb + roff[ks & 3]);
      } else {
        const int stp = (t - 4 * KS) / DB, db = (t - 4 * KS) % DB;
        opa[t] = tr_read(kt + (db >> 1) * kTileElems + 1024 * stp, troff[0][db & 1],
                         troff[1][db & 1]);
      }
    };
    // elements 2 ch, 2 ch + 1 of half kb: P = 2^(S c - L log2 e), dS = P (dP - D)
    auto probs = [&](int kb, int ch) FA_INLINE {
      float ds[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int e = 2 * ch + x;
        float sv = st[kb][e];
        if constexpr (MASK) {
          if (32 * kb + 8 * (e >> 2) + (e & 3) > lim) sv = -kInf;
        }
        const float p = fast_exp2(__builtin_fmaf(sv, c, -L2));
        if constexpr (DROP) {
          const float dpe = drop_keep(zb[kb], e, a.drop.t) ? a.drop.scale * dpt[kb][e] : 0.f;
          ds[x] = p * (dpe - Dq);
        } else {
          ds[x] = p * dpt[kb][e];
        }
      }
      pkd[2 * kb + (ch >> 2)][ch & 3] = pack2(ds[0], ds[1]);
    };

#pragma unroll
    for (int t = 0; t < kLead; ++t) load_a(t);
    FA_FENCE();
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      if (t + kLead < NS) load_a(t + kLead);
      if (t < 4 * KS) {
        const int kb = t / (2 * KS), ks = (t % (2 * KS)) >> 1;
        if (t & 1)
          dpt[kb] = mfma32(opa[t], dof[ks], dpt[kb]);
        else
          st[kb] = mfma32(opa[t], qf[ks], st[kb]);
      } else {
        const int stp = (t - 4 * KS) / DB, db = (t - 4 * KS) % DB;
        acc[db] = mfma32(opa[t], words_to_bf16x8(pkd[stp][0], pkd[stp][1], pkd[stp][2],
                                                 pkd[stp][3]), acc[db]);
      }
      if constexpr (D == 64) {
        if (t >= 8 && t < 16) probs(0, t - 8);
        if (t >= 16 && t < 20) {  // chunks 0..5 of half 1 over four slots
          probs(1, (3 * (t - 16)) >> 1);
          if ((t - 16) & 1) probs(1, ((3 * (t - 16)) >> 1) + 1);
        }
        if (t == 20 || t == 21) probs(1, t - 14);
      } else {
        // half 0 over the 2 KS slots of half 1's S^T, dP^T; half 1 over the
        // first 2 DB dQ^T slots (its first steps are needed at 4 KS + 2 DB)
        spread_chunks<2 * KS, 2 * KS>(t, [&](int cc) FA_INLINE { probs(0, cc); });
        spread_chunks<4 * KS, 2 * DB>(t, [&](int cc) FA_INLINE { probs(1, cc); });
      }
      if constexpr (DROP) {  // half t / KS, in the MFMA-only slots 0 .. 2 KS - 1
        if (t < 2 * KS) {
          const int half = t / KS, u = t % KS;
          DropBlock& z = zb[half];
          if (u == 0)
            drop_start(z, (uint32_t)((k0 >> 2) + 8 * half + 2 * (lane & 3) + hl),
                       (uint32_t)(qi >> 2), (uint32_t)bh, a.drop.offset);
          philox_rounds(z.v, a.drop.seed_lo, a.drop.seed_hi, (10 * u) / KS, (10 * (u + 1)) / KS);
          if (u == KS - 1) drop_finish<false>(z, lane);
        }
      }
      FA_FENCE();
    }
  };

  auto compute = [&](int it, const uint16_t* kt, const uint16_t* vt) FA_INLINE {
    const int k0 = tile_at(it) * kTile;
    const bool active = !CAUSAL || (k0 <= qw + 31 + a.coff);
    if (active) {
      const bool need_mask = (k0 + kTile > kv_len) || (CAUSAL && k0 + kTile - 1 > qw + a.coff);
      if (need_mask)
        body(std::true_type{}, kt, vt, k0);
      else
        body(std::false_type{}, kt, vt, k0);
    }
  };

  if (nlist > 0) stage(tile_at(0), s_k0, s_v0);
  // Every load issued so far (fragments, first tile) is complete here;
  // saying so also keeps the loop's wait counts from covering them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Two tiles per trip so that each buffer is a fixed array.
  for (int it = 0; it < nlist; it += 2) {
    if (it + 1 < nlist) stage(tile_at(it + 1), s_k1, s_v1);
    compute(it, s_k0, s_v0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 >= nlist) break;
    if (it + 2 < nlist) stage(tile_at(it + 2), s_k0, s_v0);
    compute(it + 1, s_k1, s_v1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (qi < a.N) {
    uint16_t* out = (uint16_t*)a.dq + b * a.sdq.b + hh * a.sdq.h + (int64_t)qi * a.sdq.s;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = (__bf16)(acc[db][4 * j + i] * a.scale);
        *reinterpret_cast<bf16x4*>(out + 32 * db + 8 * j + 4 * hl) = v4;
      }
  }
}

// ---------------------------------------------------------------- dK, dV

// dK, dV for the 128 keys of work item `item` (key tile, batch, head).
// s_q0/s_do0 and s_q1/s_do1 are the two Q/dO tile buffers; s_nl and s_nd
// hold -L / scale and -D of each buffer's 64 rows.  With D = 128 the
// accumulators of dK^T and dV^T take 128 registers per lane; that variant
// runs one wave per SIMD and keeps them in the accumulation registers.
template <int D, bool CAUSAL, bool SEQLEN, bool BMASK, bool DROP>
__device__ __forceinline__ void dkdv_role(const BwdArgs& a, int item, uint16_t* s_q0,
                                          uint16_t* s_do0, uint16_t* s_q1, uint16_t* s_do1,
                                          float (*s_nl)[kTile], float (*s_nd)[kTile],
                                          uint16_t* s_list, int* s_scan) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = tid >> 6;
  const int r = lane & 31, hl = lane >> 5;
  const int BH = a.B * a.H;
  constexpr int KS = D / 16;                  // contraction steps over d
  constexpr int DBo = D / 32;                 // 32-row blocks of dK^T, dV^T
  // Causal: key tile 0 sees every query, so ascending items are heaviest first.
  const int kt = item / BH;
  const int bh = item % BH;
  const int b = bh / a.H, hh = bh % a.H;
  const int k0 = kt * kBK;
  const int kw = k0 + 32 * w;  // first key of this wave
  const int kj = kw + r;       // this lane's key

  int kv_len = a.Nk;
  if constexpr (SEQLEN) kv_len = min(max(a.seqlens[b], 0), a.Nk);

  uint16_t* dK = (uint16_t*)a.dk + b * a.sdk.b + hh * a.sdk.h;
  uint16_t* dV = (uint16_t*)a.dv + b * a.sdv.b + hh * a.sdv.h;

  f32x16 dkt[DBo], dvt[DBo];
#pragma unroll
  for (int db = 0; db < DBo; ++db) dkt[db] = dvt[db] = zero16();

  if (k0 < kv_len) {
    const int nq = (a.N + kTile - 1) / kTile;
    // causal: the first query that sees key k0 is k0 - coff
    const int qt_lo = CAUSAL ? max(0, k0 - a.coff) / kTile : 0;
    int nlist = nq - qt_lo;
    [[maybe_unused]] uint16_t* tlist = nullptr;
    if constexpr (BMASK) {
      tlist = s_list;
      const int col = k0 / a.mask_block;
      nlist = build_tile_list(s_list, s_scan, a.bmask + col, a.n_mask_k, a.n_mask_q,
                              a.mask_block / kTile, qt_lo, nq);
    }

    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc((const uint16_t*)a.q + b * a.sq.b + hh * a.sq.h, slice_bytes(a.N, a.sq.s, 2, D));
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc((const uint16_t*)a.k + b * a.sk.b + hh * a.sk.h, slice_bytes(a.Nk, a.sk.s, 2, D));
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc((const uint16_t*)a.v + b * a.sv.b + hh * a.sv.h, slice_bytes(a.Nk, a.sv.s, 2, D));
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc(
        (const uint16_t*)a.dout + b * a.sdo.b + hh * a.sdo.h, slice_bytes(a.N, a.sdo.s, 2, D));
    const float* lse = a.lse + (int64_t)bh * a.N;
    const int ssq = (int)a.sq.s * 2, ssdo = (int)a.sdo.s * 2;

    // K and V fragments (B operands): lane (r, hl) holds row kj, columns
    // 16 ks + 8 hl .. +7.
    bf16x8 kf[KS], vf[KS];
    {
      const int ok = kj * (int)a.sk.s * 2 + 16 * hl;
      const int ov = kj * (int)a.sv.s * 2 + 16 * hl;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = as_bf16x8(ldb16(rk, ok + 32 * ks));
        vf[ks] = as_bf16x8(ldb16(rv, ov + 32 * ks));
      }
    }
    const float c = a.scale_log2;
    const float inv_scale = 1.f / a.scale;
    // Causal: element e of block qb holds query qs + 4*hl + off(qb, e) and is
    // visible iff off >= qs_lim - qs; keys past the sequence see nothing.
    const int key_lim =
        (kj < kv_len) ? (CAUSAL ? kj - a.coff - 4 * hl : -(1 << 30)) : (1 << 30);

    // Per-lane LDS offsets: Q and dO rows (A operands of S and dP) and Q^T,
    // dO^T transpose reads (A operands of dK^T and dV^T).
    int roff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) roff[ks] = row_off(r, hl, ks);
    int troff[2][2];
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int db = 0; db < 2; ++db) troff[hi][db] = tr_off(lane, hi, db);

    // Raw L and D of row qs + tid (threads 0..63), converted only when they
    // are written to LDS so that no wait on the loads sits at the start of a
    // tile.  Rows past N read as 0 through the buffer resources.
    float lraw = 0.f, draw = 0.f;
    int lrow = 0;
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(lse, (uint32_t)a.N * 4);
    const __amdgpu_buffer_rsrc_t rds = make_rsrc(a.dsum + (int64_t)bh * a.N, (uint32_t)a.N * 4);
    auto tile_at = [&](int it) FA_INLINE -> int {
      if constexpr (BMASK) return tlist[it];
      return qt_lo + it;
    };
    // Q and dO tiles go straight to LDS; L and D through registers.
    auto gload = [&](int t, uint16_t* qt_, uint16_t* dt_) FA_INLINE {
      const int qs = t * kTile;
#pragma unroll
      for (int j = 0; j < (D > 64 ? D / 64 : 1); ++j) {
        stage_tile(rq, qs, ssq, qt_ + j * kTileElems, w, lane, 128 * j);
        stage_tile(rdo, qs, ssdo, dt_ + j * kTileElems, w, lane, 128 * j);
      }
      if (tid < kTile) {
        lrow = qs + tid;
        lraw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * lrow, 0, 0));
        draw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rds, 4 * lrow, 0, 0));
      }
    };
    // After the loads are complete: -L / scale and -D of the tile's rows
    // (threads 0..63); the barrier that follows publishes them to every wave.
    auto swrite = [&](int buf) FA_INLINE {
      if (tid < kTile) {
        // -inf makes every probability of a dead or missing row 0
        const bool live = lrow < a.N && lraw != -kInf;
        s_nl[buf][tid] = live ? -lraw * inv_scale : -kInf;
        s_nd[buf][tid] = -draw;  // rows past N read as zeros: D = 0
      }
    };

    // One 64-query tile as 32 issue slots, each holding one MFMA, a share
    // of the vector work and the LDS reads of the operand needed kLead
    // slots later; scheduling fences keep the slots in this order so that
    // the exponentials and dS products of one 32-query half run on the
    // vector ALU while the matrix core works on the other half:
    //   slots  0.. 7  S, dP of queries 0..31                (MFMA)
    //   slots  8..15  S, dP of queries 32..63               (MFMA) | P, dS of 0..31
    //   slots 16..23  dV, dK contributions of queries 0..31 (MFMA) | P, dS of 32..63
    //   slots 24..31  dV, dK contributions of 32..63        (MFMA)
    auto tile = [&](auto mask_c, int buf, const uint16_t* qs_, const uint16_t* ds_, int qs)
        FA_INLINE {
      constexpr bool MASK = decltype(mask_c)::value;
      constexpr int kLead = 2;
      constexpr int NS = 4 * KS + 8 * DBo;  // 32 for D = 64
      f32x16 sc_[2], dp[2];
      uint32_t pkp[4][4], pkd[4][4];  // bf16 pairs of P and dS per step
      bf16x8 opa[NS];
      [[maybe_unused]] DropBlock zb[2];  // keep bytes of the two halves
      // A operand of slot t.
      auto load_a = [&](int t) FA_INLINE {
        if (t < 4 * KS) {
          const int qb = t / (2 * KS), ks = (t % (2 * KS)) >> 1;
          opa[t] = tile_row8(((t & 1) ? ds_ : qs_) + (ks >> 2) * kTileElems,
                             2048 * qb + roff[ks & 3]);
        } else {
          const int tb = t - 4 * KS;
          const int stp = tb / (2 * DBo), u = tb % (2 * DBo), db = u >> 1;
          opa[t] = tr_read(((u & 1) ? qs_ : ds_) + (db >> 1) * kTileElems + 1024 * stp,
                           troff[0][db & 1], troff[1][db & 1]);
        }
      };
      // The accumulators start at the row constants of their elements: S at
      // -L / scale and dP at -D, so the MFMAs leave S - L / scale (whose
      // product with scale log2 e is the log2 probability) and dP - D.
      auto init_acc = [&](int qb) FA_INLINE {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 32 * qb + 8 * j + 4 * hl;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&s_nl[buf][row]);
          if constexpr (DROP) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              sc_[qb][4 * j + i] = l4[i];
              dp[qb][4 * j + i] = 0.f;
            }
          } else {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(&s_nd[buf][row]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              sc_[qb][4 * j + i] = l4[i];
              dp[qb][4 * j + i] = d4[i];
            }
          }
        }
      };
      // Elements 2 ch and 2 ch + 1 of half qb: P = 2^(c (S - L / scale)),
      // dS = P (dP - D), each pair rounded to bf16.
      auto probs = [&](int qb, int ch) FA_INLINE {
        float pv[2], dv2[2];
        [[maybe_unused]] float2 nd2;
        if constexpr (DROP)  // -D of the pair's two query rows
          nd2 = *reinterpret_cast<const float2*>(
              &s_nd[buf][32 * qb + 8 * (ch >> 1) + 4 * hl + 2 * (ch & 1)]);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int e = 2 * ch + x;
          float sv = sc_[qb][e] * c;
          if constexpr (MASK) {
            if (32 * qb + 8 * (e >> 2) + (e & 3) < key_lim - qs) sv = -kInf;
          }
          pv[x] = fast_exp2(sv);
          if constexpr (DROP) {
            const bool keep = drop_keep(zb[qb], e, a.drop.t);
            const float nd = x ? nd2.y : nd2.x;
            dv2[x] = pv[x] * ((keep ? a.drop.scale * dp[qb][e] : 0.f) + nd);
            pv[x] = keep ? pv[x] : 0.f;
          } else {
            dv2[x] = dp[qb][e] * pv[x];
          }
        }
        pkp[2 * qb + (ch >> 2)][ch & 3] = pack2(pv[0], pv[1]);
        pkd[2 * qb + (ch >> 2)][ch & 3] = pack2(dv2[0], dv2[1]);
      };

      init_acc(0);
#pragma unroll
      for (int t = 0; t < kLead; ++t) load_a(t);
      FA_FENCE();
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        if (t + kLead < NS) load_a(t + kLead);
        if (t == 2) init_acc(1);
        if (t < 4 * KS) {
          const int qb = t / (2 * KS), ks = (t % (2 * KS)) >> 1;
          if (t & 1)
            dp[qb] = mfma32(opa[t], vf[ks], dp[qb]);
          else
            sc_[qb] = mfma32(opa[t], kf[ks], sc_[qb]);
        } else {
          const int tb = t - 4 * KS;
          const int stp = tb / (2 * DBo), u = tb % (2 * DBo), db = u >> 1;
          const bf16x8 bop = (u & 1) ? words_to_bf16x8(pkd[stp][0], pkd[stp][1], pkd[stp][2],
                                                       pkd[stp][3])
                                     : words_to_bf16x8(pkp[stp][0], pkp[stp][1], pkp[stp][2],
                                                       pkp[stp][3]);
          if (u & 1)
            dkt[db] = mfma32(opa[t], bop, dkt[db]);
          else
            dvt[db] = mfma32(opa[t], bop, dvt[db]);
        }
        // P, dS of half 0 over the S, dP slots of half 1, of half 1 over the
        // first half of the dV, dK slots (one chunk in each of slots 8..23 for
        // D = 64)
        if constexpr (D == 64) {
          if (t >= 8 && t < 24) probs((t - 8) >> 3, (t - 8) & 7);
        } else {
          spread_chunks<2 * KS, 2 * KS>(t, [&](int cc) FA_INLINE { probs(0, cc); });
          spread_chunks<4 * KS, 4 * DBo>(t, [&](int cc) FA_INLINE { probs(1, cc); });
        }
        if constexpr (DROP) {  // half t / KS, in slots 0 .. 2 KS - 1
          if (t < 2 * KS) {
            const int half = t / KS, u = t % KS;
            DropBlock& z = zb[half];
            if (u == 0)
              drop_start(z, (uint32_t)(kj >> 2),
                         (uint32_t)((qs >> 2) + 8 * half + 2 * (lane & 3) + hl),
                         (uint32_t)bh, a.drop.offset);
            philox_rounds(z.v, a.drop.seed_lo, a.drop.seed_hi, (10 * u) / KS,
                          (10 * (u + 1)) / KS);
            if (u == KS - 1) drop_finish<true>(z, lane);
          }
        }
        FA_FENCE();
      }
    };

    auto compute = [&](int it, int buf, const uint16_t* qs_, const uint16_t* ds_) FA_INLINE {
      const int qs = tile_at(it) * kTile;
      const bool active = !CAUSAL || (qs + kTile - 1 >= kw - a.coff);
      if (active) {
        const bool need_mask = (kw + 32 > kv_len) || (CAUSAL && kw + 31 - a.coff > qs);
        if (need_mask)
          tile(std::true_type{}, buf, qs_, ds_, qs);
        else
          tile(std::false_type{}, buf, qs_, ds_, qs);
      }
    };

    if (nlist > 0) {
      gload(tile_at(0), s_q0, s_do0);
      __builtin_amdgcn_s_waitcnt(0);
      swrite(0);
    }
    // Every load issued so far (K, V fragments, first tile) is complete here;
    // saying so also keeps the loop's wait counts from covering them.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Two tiles per trip so that each buffer is a fixed array.
    for (int it = 0; it < nlist; it += 2) {
      if (it + 1 < nlist) gload(tile_at(it + 1), s_q1, s_do1);
      compute(it, 0, s_q0, s_do0);
      __builtin_amdgcn_s_waitcnt(0);
      if (it + 1 < nlist) swrite(1);
      __syncthreads();
      if (it + 1 >= nlist) break;
      if (it + 2 < nlist) gload(tile_at(it + 2), s_q0, s_do0);
      compute(it + 1, 1, s_q1, s_do1);
      __builtin_amdgcn_s_waitcnt(0);
      if (it + 2 < nlist) swrite(0);
      __syncthreads();
    }
  }

  if (kj < a.Nk) {
    uint16_t* kout = dK + (int64_t)kj * a.sdk.s;
    uint16_t* vout = dV + (int64_t)kj * a.sdv.s;
#pragma unroll
    for (int db = 0; db < DBo; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 k4, v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          k4[i] = (__bf16)(dkt[db][4 * j + i] * a.scale);
          v4[i] = (__bf16)(DROP ? dvt[db][4 * j + i] * a.drop.scale : dvt[db][4 * j + i]);
        }
        *reinterpret_cast<bf16x4*>(kout + 32 * db + 8 * j + 4 * hl) = k4;
        *reinterpret_cast<bf16x4*>(vout + 32 * db + 8 * j + 4 * hl) = v4;
      }
  }
}

// The fused backward kernel.  Work items: query tiles for the dQ role and
// key tiles for the dK/dV role (each times B*H), each role in its own
// heavy-first order.
// D = 32, 64: two waves per SIMD are asked for explicitly: left to itself the
// compiler gives some dropout variants 256 VGPRs plus AGPR spill slots (one
// wave per SIMD, a third slower); with the bound they fit in 256 registers,
// and the other variants compile unchanged.  D = 128 runs one wave per SIMD:
// its dK/dV accumulators alone take 128 registers per lane, and its
// translation unit keeps them in the accumulation registers.
template <int D, bool CAUSAL, bool SEQLEN, bool BMASK, bool DROP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 8))) void bwd_kernel(
    BwdArgs a, int phases) {
  constexpr int KB = D > 64 ? D / 64 : 1;   // 64-column blocks per LDS tile
  // Four tile arrays, two per buffer: K and V in the dQ role, Q and dO in
  // the dK/dV role.  Separate arrays, so that the copies into one buffer and
  // the reads of the other never alias.
  __shared__ __attribute__((aligned(16))) uint16_t s_a0[KB * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t s_b0[KB * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t s_a1[KB * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t s_b1[KB * kTileElems];
  __shared__ __attribute__((aligned(16))) float s_nl[2][kTile];  // -L / scale
  __shared__ __attribute__((aligned(16))) float s_nd[2][kTile];  // -D
  __shared__ uint16_t s_list[BMASK ? kMaxListTiles : 1];
  __shared__ int s_scan[4];

  // Workgroup ids go to the 8 XCDs round robin.  With B*H a multiple of 8,
  // ids are mapped so that every work item of one (batch, head) -- both
  // roles -- runs on the same XCD and shares its L2: XCD x serves the heads
  // x, x + 8, ...; it takes all its dK/dV tiles before its dQ tiles, so
  // that mostly one role runs at a time (mixing them grows the working set
  // each L2 has to hold: item by item it measured 6-20 % slower) while the
  // switch from one to the other and the tail still overlap.  Within a role
  // the causal items go heaviest first, walking the heads fastest; without
  // the causal mask the items weigh the same, and the XCD's heads are taken
  // in groups of 4, each group's tiles before the next group's, so that
  // fewer heads' tiles compete for L2 at a time (BERT-large shape: 76 ->
  // 71 us; the causal 1K shape measured 2 % slower grouped, its balance
  // matters more).  Items are numbered tile * B*H + (batch, head), as the
  // roles expect.  (Dealing the
  // causal items to the CUs in snake order, as the forward does, measured
  // 3-5 % slower here: with two items resident per CU and the rest
  // dispatched as CUs free up, heaviest first is already balanced.)
  const int id = blockIdx.x;
  const int BH = a.B * a.H;
  bool dkdv;
  int item;
  if (phases == (kPhaseDQ | kPhaseDKDV)) {
    // The role whose items are heavier goes first: a dK/dV item sweeps the
    // queries, a dQ item the keys.
    const bool dq_first = a.Nk > a.N;
    const int nfirst = dq_first ? (a.N + kBQ - 1) / kBQ : (a.Nk + kBK - 1) / kBK;
    bool first;
    if ((BH & 7) == 0) {
      const int hpx = BH >> 3, x = id & 7, j = id >> 3;  // hpx heads per XCD
      const int nsecond = dq_first ? (a.Nk + kBK - 1) / kBK : (a.N + kBQ - 1) / kBQ;
      first = j < nfirst * hpx;
      const int jr = first ? j : j - nfirst * hpx;  // rank within the role
      const int nt = first ? nfirst : nsecond;       // tiles per head
      const int hg = CAUSAL ? hpx : 4;               // heads per group
      const int gi = jr / (hg * nt), within = jr % (hg * nt);
      const int gsize = min(hg, hpx - gi * hg);      // the last group may be smaller
      item = (within / gsize) * BH + x + 8 * (gi * hg + within % gsize);
    } else {
      first = id < nfirst * BH;
      item = first ? id : id - nfirst * BH;
    }
    dkdv = first != dq_first;
  } else {
    dkdv = phases == kPhaseDKDV;
    item = id;
  }
  if (dkdv)
    dkdv_role<D, CAUSAL, SEQLEN, BMASK, DROP>(a, item, s_a0, s_b0, s_a1, s_b1, s_nl, s_nd,
                                              s_list, s_scan);
  else
    dq_role<D, CAUSAL, SEQLEN, BMASK, DROP>(a, item, s_a0, s_b0, s_a1, s_b1, s_list, s_scan);
}

// D_i = dot(dO_i, O_i) of every query row into a.dsum (fp32 [B*H*N]): 64
// rows per workgroup, four threads per row, each taking a quarter of the
// row's D elements in 16-byte loads (rows are 16-byte aligned).
template <int D>
__global__ __launch_bounds__(256) void dsum_kernel(BwdArgs a) {
  const int tid = threadIdx.x;
  const int nrt = (a.N + 63) / 64;
  const int bh = blockIdx.x / nrt, rt = blockIdx.x % nrt;
  const int b = bh / a.H, hh = bh % a.H;
  const int row = rt * 64 + (tid >> 2), part = tid & 3;
  float acc = 0.f;
  if (row < a.N) {
    const uint16_t* dop = (const uint16_t*)a.dout + b * a.sdo.b + hh * a.sdo.h +
                          (int64_t)row * a.sdo.s + part * (D / 4);
    const uint16_t* op =
        (const uint16_t*)a.o + b * a.so.b + hh * a.so.h + (int64_t)row * a.so.s + part * (D / 4);
#pragma unroll
    for (int c = 0; c < D / 4; c += 8)
      acc = dot8_bf16(*reinterpret_cast<const bf16x8*>(dop + c),
                      *reinterpret_cast<const bf16x8*>(op + c), acc);
  }
  acc += quad_xor1(acc);
  acc += quad_xor2(acc);
  if (part == 0 && row < a.N) a.dsum[(int64_t)bh * a.N + row] = acc;
}

template <int HD, bool C, bool S, bool M, bool D>
hipError_t launch(const BwdArgs& a, int phases, hipStream_t stream) {
  {
    BwdArgs c = a;
    void* args[] = {&c};
    const int nrt = (a.N + 63) / 64;
    const hipError_t e =
        hipLaunchKernel((const void*)&dsum_kernel<HD>, dim3((unsigned)(nrt * a.B * a.H)),
                        dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  BwdArgs copy = a;
  int ph = phases;
  void* args[] = {&copy, &ph};
  const int n_dq = ((a.N + kBQ - 1) / kBQ) * a.B * a.H;
  const int n_dkdv = ((a.Nk + kBK - 1) / kBK) * a.B * a.H;
  int n = 0;
  if (phases & kPhaseDQ) n += n_dq;
  if (phases & kPhaseDKDV) n += n_dkdv;
  if (n == 0) return hipSuccess;
  return hipLaunchKernel((const void*)&bwd_kernel<HD, C, S, M, D>, dim3((unsigned)n),
                         dim3(256), args, 0, stream);
}

template <int HD, bool D>
hipError_t dispatch(const BwdArgs& a, bool causal, int p, hipStream_t stream) {
  const bool s = a.seqlens != nullptr, m = a.bmask != nullptr;
  if (causal) {
    if (s)
      return m ? launch<HD, true, true, true, D>(a, p, stream)
               : launch<HD, true, true, false, D>(a, p, stream);
    return m ? launch<HD, true, false, true, D>(a, p, stream)
             : launch<HD, true, false, false, D>(a, p, stream);
  }
  if (s)
    return m ? launch<HD, false, true, true, D>(a, p, stream)
             : launch<HD, false, true, false, D>(a, p, stream);
  return m ? launch<HD, false, false, true, D>(a, p, stream)
           : launch<HD, false, false, false, D>(a, p, stream);
}

}  // namespace
}  // namespace fa
