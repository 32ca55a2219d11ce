// Fused attention forward for gfx950, bf16 inputs, fp32 accumulation.
//
// One workgroup (4 waves) owns 128 query rows of one (batch, head); each wave
// owns 32 of them and keeps its Q fragment in registers for the whole kernel.
// (Workgroups of 2 or 8 waves, 64 or 256 query rows, are also built: the
// query tile height sets how often K and V are streamed, the quantity in the
// pages' IO analysis -- researchpapers.dev, "tiling and recomputation".)
// Key/value tiles of 64 rows stream through LDS, double-buffered and copied
// straight from memory into LDS (the copy of tile t+1 is in flight while
// tile t is computed), so each K/V element is read from HBM/L2 once per
// workgroup and the N x N score matrix never leaves registers (suanlizi.com
// summary, "tiling" and "kernel fusion"; researchpapers.dev explainer,
// "tiling and recomputation").
//
// The scores are computed transposed, S^T = K Q^T, on the 32x32x16 bf16 MFMA:
// in the accumulator layout each lane then holds 32 scores of a single query
// (the two wave halves hold its two interleaved key halves).  O^T = V^T P^T is
// accumulated on the same MFMA; the probabilities feed the B operand straight
// from the accumulator registers and the V^T operand comes from the V tile
// through LDS transpose reads.
//
// Online softmax (researchpapers.dev, "tiling and recomputation"; the maximum
// subtraction is the safe softmax of the llm-deploy note).  Each query keeps
// a reference maximum m (log2 units) and a running sum l, and the output is
// O = acc / l, L = (m + log2 l) ln 2 -- a ratio that does not depend on which
// reference was used, so m only has to bound the scores, not equal their
// maximum.  Probabilities of each 32-key half tile are computed against the
// current m; if some lane's partial sum exceeds 2^12 (or is not finite, as on
// the first tile where m = -inf) every probability of that half may be too
// large, and only then is the half's true maximum taken, m raised, acc and l
// rescaled and the half recomputed.  In steady state no row maximum is
// computed at all.
//
// Tiles that the mask removes entirely are never loaded: causal and key
// padding shrink the key range, and a block mask is compacted into a list of
// kept tiles (suanlizi.com, "block-sparse attention").
//
// There is one instantiation for causal and non-causal calls: key j is
// visible to query i iff j <= i + coff, and a non-causal call passes
// coff = Nk, for which every key passes.  The extra compares cost nothing
// measurable, while a separately compiled non-causal kernel took 182 VGPRs
// (two waves per SIMD) against 160 (three): the shared one runs the dense
// and block-sparse forward 8-26 % faster.
//
// Dropout (DROP): the pages count dropout among the element-wise operations
// the fused kernel absorbs (suanlizi.com, per-component timing figure of
// "kernel fusion").  The keep bytes of each 32-key half come from one Philox
// call per lane, run in the MFMA-only slots before the half's probabilities
// are formed; a dropped probability still counts in l (L is the statistic of
// the undropped softmax) but enters O^T += V^T P^T as zero, and the keep
// scale is applied with 1 / l at the end.
#include <atomic>
#include <type_traits>

#include "fa_device.h"

namespace fa {
namespace {

// Key-range groups of a split query tile: as many 4-wave groups as the
// registers allow at three (d <= 64) or two (d = 128) waves per SIMD.
constexpr int groups_for_d(int d) { return d == 128 ? 2 : 3; }

constexpr float kSumLimit = 4096.f;    // largest partial sum the fast path accepts

// W waves, 32 W query rows per workgroup; head dimension D = 32, 64 or 128.
// A K or V tile of 64 rows is held as KB = max(1, D / 64) swizzled 64 x 64
// blocks (columns 64 j .. 64 j + 63 in block j; with D = 32 only the first
// four chunks of each row are used), so every LDS read keeps the
// conflict-free pattern of the 64-column tile.
// The 4-wave D = 64 kernels are held to three waves per SIMD (168 VGPRs):
// the variants without dropout need 160-162, the dropout ones 165, which
// measured 7-10 % faster than their 172-register, two-wave build.  So are the
// 2-wave ones without a block mask (with it, LDS allows fewer workgroups).
//
// G > 1 splits the key range of the query tile over G groups of W waves
// (group g takes the g-th of G equal runs of the tile list, each with its
// own K/V buffers); at the end the groups' (m, l, acc) are merged through
// LDS by the online-softmax rescaling and group 0 writes the outputs.  It is
// used when the grid has no more query tiles than the GPU has CUs, where a
// single group would leave one wave per SIMD.
template <int W, int G, int D, bool SEQLEN, bool BMASK, bool DROP>
__global__ __launch_bounds__(64 * W * G) __attribute__((amdgpu_waves_per_eu((D == 64 && (W == 4 || (W == 2 && !BMASK))) ? 3 : 1, 8))) void fwd_bf16_kernel(FwdArgs a) {
  static_assert(D == 32 || D == 64 || D == 128, "head dimension 32, 64 or 128");
  constexpr int kBR = 32 * W;
  constexpr int KB = D > 64 ? D / 64 : 1;  // 64-column blocks per tile
  constexpr int KS = D / 16;               // contraction steps of S^T; slots per phase
  constexpr int DB = D / 32;               // 32-row blocks of O^T
  constexpr int LEAD = KS < 4 ? KS : 4;    // slots between an operand's read and its use
  static_assert(G == 1 || (W == 4 && G <= 3), "key-range groups of 4 waves");
  // Two buffers per group, each a K tile and a V tile; separate arrays so
  // that the copies into one buffer and the reads of the other never alias.
  __shared__ __attribute__((aligned(16))) uint16_t s_k0g[G][KB * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t s_v0g[G][KB * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t s_k1g[G][KB * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t s_v1g[G][KB * kTileElems];

  const int tid = threadIdx.x, lane = tid & 63;
  // key-range group (uniform in a wave: read from the first lane)
  const int g = G > 1 ? __builtin_amdgcn_readfirstlane((tid >> 6) / W) : 0;
  const int w = G > 1 ? (tid >> 6) % W : tid >> 6;  // wave within the group
  uint16_t* const s_k0 = s_k0g[g];
  uint16_t* const s_v0 = s_v0g[g];
  uint16_t* const s_k1 = s_k1g[g];
  uint16_t* const s_v1 = s_v1g[g];
  const int r = lane & 31, hl = lane >> 5;
  const int BH = a.B * a.H;
  const int nqt = (a.N + kBR - 1) / kBR;
  // The longest query tiles (causal) are dispatched first; with four waves
  // (two or three workgroups resident per CU) they are dealt to the CUs of
  // an XCD in snake order, which measured 1-5 % faster there and slower for
  // the 2- and 8-wave workgroups.  Consecutive ids walk the heads, so with
  // B*H a multiple of 8 all tiles of one head land on the same XCD and share
  // its L2.
  const int id = W == 4 ? snake_id(blockIdx.x, gridDim.x) : blockIdx.x;
  const int qt = nqt - 1 - id / BH;
  const int bh = id % BH;
  const int b = bh / a.H, hh = bh % a.H;
  const int q0 = qt * kBR;
  const int qw = q0 + 32 * w;  // first query of this wave
  const int qi = qw + r;       // this lane's query

  int kv_len = a.Nk;
  if constexpr (SEQLEN) kv_len = min(max(a.seqlens[b], 0), a.Nk);
  const int kend = max(0, min(kv_len, q0 + kBR + a.coff));
  const int ntk = (kend + kTile - 1) / kTile;

  int nlist = ntk;
  [[maybe_unused]] uint16_t* tlist = nullptr;
  if constexpr (BMASK) {
    __shared__ uint16_t s_list[kMaxListTiles];
    __shared__ int s_scan[W * G];
    tlist = s_list;
    const int row = q0 / a.mask_block;  // the host makes the query tile divide mask_block
    nlist = build_tile_list<64 * W * G>(s_list, s_scan, a.bmask + (int64_t)row * a.n_mask_k, 1,
                                        a.n_mask_k, a.mask_block / kTile, 0, ntk);
  }
  // This group's run of the tile list, and the trips every group makes (the
  // barriers of all groups have to match).
  const int lo = G > 1 ? g * nlist / G : 0;
  const int cnt = G > 1 ? (g + 1) * nlist / G - lo : nlist;
  const int trips = G > 1 ? (nlist + G - 1) / G : nlist;

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(
      (const uint16_t*)a.q + b * a.sq.b + hh * a.sq.h, slice_bytes(a.N, a.sq.s, 2, D));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(
      (const uint16_t*)a.k + b * a.sk.b + hh * a.sk.h, slice_bytes(a.Nk, a.sk.s, 2, D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(
      (const uint16_t*)a.v + b * a.sv.b + hh * a.sv.h, slice_bytes(a.Nk, a.sv.s, 2, D));
  const int ssk = (int)a.sk.s * 2, ssv = (int)a.sv.s * 2;

  // Q fragment: B operand of S^T = K Q^T, lane (r, hl) holds
  // Q[qi][16 ks + 8 hl .. +7].  Rows past N read as zeros.
  bf16x8 qf[KS];
  {
    const int off = qi * (int)a.sq.s * 2 + 16 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(ldb16(rq, off + 32 * ks));
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();
  float m = -kInf, l = 0.f;
  const float c = a.scale_log2;

  // Per-lane LDS offsets: K rows (A operand of S^T, contraction over d) and
  // V^T transpose reads (A operand of O^T, contraction over keys).
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
    // The tile index is made opaque (an empty asm that claims to change the
    // uniform register holding it), so that the compiler recomputes the
    // tile's addresses and dropout counters from it instead of keeping
    // loop-carried copies: without it the dropout kernels need 2 registers
    // more than three waves per SIMD allow.
    int t = it;
    __asm__ volatile("" : "+s"(t));
    return t;
  };
  auto stage = [&](int t, uint16_t* kt, uint16_t* vt) FA_INLINE {
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      stage_tile<W>(rk, t * kTile, ssk, kt + j * kTileElems, w, lane, 128 * j);
      stage_tile<W>(rv, t * kTile, ssv, vt + j * kTileElems, w, lane, 128 * j);
    }
  };

  // Raises m to cover the scores of half kb, rescales acc and l, and
  // recomputes the half's probabilities (the rare path of the online softmax).
  auto rescale_to = [&](const f32x16& sv) FA_INLINE {
    float mx = -kInf;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sv[e]);
    const float mt = half_max(mx) * c;
    const float m_new = fmaxf(m, mt);
    const float alpha = (m_new == m) ? 1.f : fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
    m = m_new;
  };

  // One 64-key tile as 4 KS MFMA issue slots (16 for D = 64) in four phases
  // of KS slots, separated by scheduling fences:
  //   phase 0  S^T of keys  0..31, KS steps             (MFMA) | [keep bytes]
  //   phase 1  S^T of keys 32..63                       (MFMA) | P of keys 0..31
  //   phase 2  O^T += V^T P^T, keys 0..31: 2 x DB steps (MFMA) | P of keys 32..63
  //   phase 3  O^T += V^T P^T, keys 32..63              (MFMA)
  // Each slot issues the LDS read of the operand LEAD slots ahead (for
  // D <= 64 the same position of the next phase); the first LEAD operands are
  // read before the first slot.
  auto body = [&](auto mask_c, const uint16_t* kt, const uint16_t* vt, int k0) FA_INLINE {
    constexpr bool MASK = decltype(mask_c)::value;
    f32x16 s[2] = {zero16(), zero16()};
    bf16x8 opa[4 * KS];  // A operand of each slot
    uint32_t pk[4][4];   // bf16 pairs of P for PV steps 0..3
    float ps[2] = {0.f, 0.f};
    [[maybe_unused]] DropBlock zb[2];  // keep bytes of the two halves
    // element e of half kb holds key k0 + 32 kb + 8 (e / 4) + 4 hl + e % 4;
    // visible iff 32 kb + 8 (e / 4) + e % 4 <= lim
    [[maybe_unused]] int lim = 0;
    if constexpr (MASK) lim = min(kv_len - 1, qi + a.coff) - k0 - 4 * hl;

    auto probs = [&](int kb, int e0) FA_INLINE {  // elements e0 .. e0+3 of half kb
      float p[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int e = e0 + x;
        float sv = s[kb][e];
        if constexpr (MASK) {
          if (32 * kb + 8 * (e >> 2) + (e & 3) > lim) sv = -kInf;
        }
        p[x] = fast_exp2(__builtin_fmaf(sv, c, -m));
        ps[kb] = (e == 0) ? p[x] : ps[kb] + p[x];  // the first term starts the sum
        if constexpr (DROP) p[x] = drop_keep(zb[kb], e, a.drop.t) ? p[x] : 0.f;
      }
      const int st = 2 * kb + (e0 >> 3), wd = (e0 & 7) >> 1;
      pk[st][wd] = pack2(p[0], p[1]);
      pk[st][wd + 1] = pack2(p[2], p[3]);
    };
    // the rare path: true maximum of half kb, rescale, recompute its P
    auto fix_half = [&](int kb) FA_INLINE {
      if constexpr (MASK) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * kb + 8 * (e >> 2) + (e & 3) > lim) s[kb][e] = -kInf;
      }
      rescale_to(s[kb]);
      const float m_use = (m == -kInf) ? 0.f : m;
      ps[kb] = 0.f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        float p0 = fast_exp2(__builtin_fmaf(s[kb][e], c, -m_use));
        float p1 = fast_exp2(__builtin_fmaf(s[kb][e + 1], c, -m_use));
        ps[kb] += p0 + p1;
        if constexpr (DROP) {
          p0 = drop_keep(zb[kb], e, a.drop.t) ? p0 : 0.f;
          p1 = drop_keep(zb[kb], e + 1, a.drop.t) ? p1 : 0.f;
        }
        pk[2 * kb + (e >> 3)][(e & 7) >> 1] = pack2(p0, p1);
      }
    };

    // A operand of slot t: K rows (phases 0, 1) or V^T transpose reads
    // (phases 2, 3: key step st, output block db).
    auto load_a = [&](int t) FA_INLINE {
      const int ph = t / KS, i = t % KS;
      if (ph < 2) {
        opa[t] = tile_row8(kt + (i >> 2) * kTileElems, 2048 * ph + roff[i & 3]);
      } else {
        const int st = 2 * (ph - 2) + i / DB, db = i % DB;
        opa[t] = tr_read(vt + (db >> 1) * kTileElems + 1024 * st, troff[0][db & 1],
                         troff[1][db & 1]);
      }
    };

#pragma unroll
    for (int t = 0; t < LEAD; ++t) load_a(t);
    FA_FENCE();
#pragma unroll
    for (int t = 0; t < 4 * KS; ++t) {
      const int ph = t / KS, i = t % KS;
      if (ph < 2) {
        s[ph] = mfma32(opa[t], qf[i], s[ph]);
      } else {
        const int st = 2 * (ph - 2) + i / DB, db = i % DB;
        o[db] = mfma32(opa[t], words_to_bf16x8(pk[st][0], pk[st][1], pk[st][2], pk[st][3]),
                       o[db]);
      }
      if (t + LEAD < 4 * KS) load_a(t + LEAD);
      if constexpr (DROP) {  // half i / (KS / 2), its ten rounds over KS / 2 slots
        if (ph == 0) {
          constexpr int NSUB = KS / 2;
          const int half = i / NSUB, u = i % NSUB;
          DropBlock& z = zb[half];
          if (u == 0)
            drop_start(z, (uint32_t)((k0 >> 2) + 8 * half + 2 * (lane & 3) + hl),
                       (uint32_t)(qi >> 2), (uint32_t)bh, a.drop.offset);
          philox_rounds(z.v, a.drop.seed_lo, a.drop.seed_hi, (10 * u) / NSUB,
                        (10 * (u + 1)) / NSUB);
          if (u == NSUB - 1) drop_finish<false>(z, lane);
        }
      }
      if (ph == 1 || ph == 2) {  // P of half ph - 1, four elements per call
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
          if ((cc * KS) / 4 == i) probs(ph - 1, 4 * cc);
      }
      FA_FENCE();
      if (t == 2 * KS - 1 || t == 3 * KS - 1) {
        const int kb = (t == 2 * KS - 1) ? 0 : 1;
        if (__any(!(ps[kb] <= kSumLimit))) fix_half(kb);
        l += ps[kb];
        FA_FENCE();
      }
    }
  };

  auto compute = [&](int it, const uint16_t* kt, const uint16_t* vt) FA_INLINE {
    const int k0 = tile_at(it) * kTile;
    const bool active = k0 <= qw + 31 + a.coff;
    if (active) {
      const bool need_mask = (k0 + kTile > kv_len) || (k0 + kTile - 1 > qw + a.coff);
      if (need_mask)
        body(std::true_type{}, kt, vt, k0);
      else
        body(std::false_type{}, kt, vt, k0);
    }
  };

  if (cnt > 0) stage(tile_at(lo), s_k0, s_v0);
  // Every load issued so far (Q fragment, first tile) is complete here;
  // saying so also keeps the loop's wait counts from covering them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Two tiles per trip so that each buffer is a fixed array.
  for (int it = 0; it < trips; it += 2) {
    if (it + 1 < cnt) stage(tile_at(lo + it + 1), s_k1, s_v1);
    if (G == 1 || it < cnt) compute(lo + it, s_k0, s_v0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 >= trips) break;
    if (it + 2 < cnt) stage(tile_at(lo + it + 2), s_k0, s_v0);
    if (G == 1 || it + 1 < cnt) compute(lo + it + 1, s_k1, s_v1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if constexpr (G > 1) {
    // Groups 1 .. G-1 hand their state to group 0 one at a time, through the
    // K/V buffers (free: every read of them completed before the last
    // barrier).  Per wave and lane: acc block db in s_k0g (db < max(1, DB/2))
    // or s_v0g, then m and l in s_k1g, each float at [element][wave][lane].
    float* const xo0 = reinterpret_cast<float*>(&s_k0g[0][0]);
    float* const xo1 = reinterpret_cast<float*>(&s_v0g[0][0]);
    float* const xml = reinterpret_cast<float*>(&s_k1g[0][0]);
    constexpr int kHalf = DB > 1 ? DB / 2 : 1;  // acc blocks in xo0
    constexpr int kBufBytes = G * KB * kTileElems * 2;  // bytes of each buffer array
    static_assert(kHalf * 16 * 64 * W * 4 <= kBufBytes, "acc blocks fit the buffers");
    static_assert(2 * 64 * W * 4 <= kBufBytes, "m and l fit a buffer");
    const int slot = w * 64 + lane;            // this lane's column
    auto at = [&](int db, int e) FA_INLINE -> float* {
      float* base = db < kHalf ? xo0 : xo1;
      return base + ((db % kHalf) * 16 + e) * (64 * W) + slot;
    };
#pragma unroll
    for (int j = 1; j < G; ++j) {
      if (g == j) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) *at(db, e) = o[db][e];
        xml[slot] = m;
        xml[64 * W + slot] = l;
      }
      __syncthreads();
      if (g == 0) {
        const float mj = xml[slot], lj = xml[64 * W + slot];
        const float m_new = fmaxf(m, mj);
        // a dead side (m = -inf, l = 0, acc = 0) gets weight 0, or 1 if both are
        const float a0 = (m == m_new) ? 1.f : fast_exp2(m - m_new);
        const float aj = (mj == m_new) ? 1.f : fast_exp2(mj - m_new);
        l = l * a0 + lj * aj;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][e] = o[db][e] * a0 + *at(db, e) * aj;
        m = m_new;
      }
      __syncthreads();
    }
    if (g != 0) return;
  }

  const float lt = half_sum(l);
  if (qi < a.N) {
    float inv = lt > 0.f ? 1.f / lt : 0.f;
    if constexpr (DROP) inv *= a.drop.scale;
    uint16_t* op = (uint16_t*)a.o + b * a.so.b + hh * a.so.h + (int64_t)qi * a.so.s;
#pragma unroll
    for (int db = 0; db < DB; ++db)
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

template <int W, int G, int HD, bool S, bool M, bool D>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.N + 32 * W - 1) / (32 * W);
  dim3 grid((unsigned)(nqt * a.B * a.H)), block(64 * W * G);
  FwdArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel((const void*)&fwd_bf16_kernel<W, G, HD, S, M, D>, grid, block, args,
                         0, stream);
}

template <int W, int G, int HD, bool D>
hipError_t dispatch_masks(const FwdArgs& c, hipStream_t stream) {
  const bool s = c.seqlens != nullptr, m = c.bmask != nullptr;
  if (s)
    return m ? launch<W, G, HD, true, true, D>(c, stream)
             : launch<W, G, HD, true, false, D>(c, stream);
  return m ? launch<W, G, HD, false, true, D>(c, stream)
           : launch<W, G, HD, false, false, D>(c, stream);
}

// Non-causal calls run with the causal offset Nk, which makes every key
// visible to every query.
template <int W, int HD, bool D, int GS = 1>
hipError_t dispatch(const FwdArgs& a, bool causal, hipStream_t stream) {
  FwdArgs c = a;
  if (!causal) c.coff = a.Nk;
  if constexpr (GS > 1) {
    if (fwd_key_groups(a.B, a.H, a.N, a.Nk, HD, 32 * W) > 1)
      return dispatch_masks<W, GS, HD, D>(c, stream);
  }
  return dispatch_masks<W, 1, HD, D>(c, stream);
}

}  // namespace

// CUs of the current device (0 if it cannot be read: no split then), read
// from the runtime once per device and kept in a small table.
static int cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];  // 0: not read yet
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices && (n = cached[dev].load(std::memory_order_relaxed)) > 0)
    return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev >= 0 && dev < kMaxDevices && n > 0) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int fwd_key_groups(int B, int H, int N, int Nk, int d, int block_q) {
  if (block_q != 128 || Nk < 1024) return 1;
  const long items = (long)((N + 127) / 128) * B * H;
  if (items > cu_count()) return 1;
  return groups_for_d(d);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, bool causal, int block_q, int d,
                           hipStream_t stream) {
  // the host allows dropout and d != 64 only with block_q = 128
  const bool drop = a.drop.t < 256;
  if (d == 32)
    return drop ? dispatch<4, 32, true, groups_for_d(32)>(a, causal, stream)
                : dispatch<4, 32, false, groups_for_d(32)>(a, causal, stream);
  if (d == 128)
    return drop ? dispatch<4, 128, true, groups_for_d(128)>(a, causal, stream)
                : dispatch<4, 128, false, groups_for_d(128)>(a, causal, stream);
  if (drop) return dispatch<4, 64, true, groups_for_d(64)>(a, causal, stream);
  if (block_q == 64) return dispatch<2, 64, false>(a, causal, stream);
  if (block_q == 256) return dispatch<8, 64, false>(a, causal, stream);
  return dispatch<4, 64, false, groups_for_d(64)>(a, causal, stream);
}

}  // namespace fa
