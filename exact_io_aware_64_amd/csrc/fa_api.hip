// Host side of the C ABI declared in include/fa.h: argument validation,
// launch-argument packing and dispatch.  Validation finishes before the
// first HIP call, so rejected calls never touch the device.
#include "../../include/fa.h"

#include <math.h>
#include <stdarg.h>

#include <mutex>
#include <stdio.h>
#include <string.h>

#include "fa_internal.h"

namespace {

thread_local char g_err[512] = "";

fa_status fail(fa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

fa_status check_tensor(const char* name, const void* p, fa_strides s, int elem_align, int N) {
  if (p == nullptr) return fail(FA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(FA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  if (s.batch < 0 || s.head < 0 || s.seq < 0)
    return fail(FA_ERR_INVALID_ARG, "%s has a negative stride", name);
  if (s.batch % elem_align || s.head % elem_align || s.seq % elem_align)
    return fail(FA_ERR_INVALID_ARG, "%s strides must be multiples of %d elements", name,
                elem_align);
  // The kernels address one (batch, head) slice with 32-bit byte offsets,
  // including up to 128 rows past its end.
  const int esize = elem_align == 8 ? 2 : 4;
  if (((long long)N + 128) * (long long)s.seq * esize >= (1LL << 31))
    return fail(FA_ERR_UNSUPPORTED, "%s: one (batch, head) slice spans 2 GiB or more", name);
  return FA_OK;
}

fa_status check_common(fa_dtype dtype, int B, int H, int N, int Nk, int d, float scale,
                       const uint8_t* block_mask, int mask_block, int* elem_align) {
  if (dtype != FA_BF16 && dtype != FA_F32)
    return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B <= 0 || H <= 0 || N <= 0)
    return fail(FA_ERR_INVALID_ARG, "B, H and N must be positive (got %d, %d, %d)", B, H, N);
  if (Nk <= 0) return fail(FA_ERR_INVALID_ARG, "N_k must be positive (got %d)", Nk);
  if (d != 32 && d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dimension %d is not supported (32, 64, 128)", d);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(FA_ERR_INVALID_ARG, "scale must be positive and finite");
  const long long tiles = ((long long)(N > Nk ? N : Nk) + fa::kTile - 1) / fa::kTile;
  if (2 * tiles * (long long)B * H > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "problem too large for one launch grid");
  if (block_mask != nullptr) {
    if (mask_block <= 0 || mask_block % 128 != 0)
      return fail(FA_ERR_INVALID_ARG, "mask_block must be a positive multiple of 128 (got %d)",
                  mask_block);
    if (tiles > fa::kMaxListTiles)
      return fail(FA_ERR_UNSUPPORTED, "block mask supports N, N_k <= %d",
                  fa::kMaxListTiles * 64);
  }
  *elem_align = dtype == FA_BF16 ? 8 : 4;
  return FA_OK;
}

fa::Strides cvt(fa_strides s) { return fa::Strides{s.batch, s.head, s.seq}; }

// Keep threshold t = floor(256 (1 - p) + 1/2), computed in double; p = 0
// gives t = 256 (keep every pair).
fa_status make_dropout(float p, uint64_t seed, uint32_t offset, fa::Dropout* d) {
  if (!(p >= 0.f && p < 1.f))
    return fail(FA_ERR_INVALID_ARG, "dropout_p must lie in [0, 1) (got %g)", (double)p);
  const int t = (int)floor(256.0 * (1.0 - (double)p) + 0.5);
  if (t < 1)
    return fail(FA_ERR_INVALID_ARG, "dropout_p %g rounds to dropping every pair", (double)p);
  d->t = (uint32_t)t;
  d->scale = (float)(256.0 / t);
  d->seed_lo = (uint32_t)seed;
  d->seed_hi = (uint32_t)(seed >> 32);
  d->offset = offset;
  return FA_OK;
}

fa_status hip_status(hipError_t e) {
  if (e == hipSuccess) {
    g_err[0] = '\0';
    return FA_OK;
  }
  return fail(FA_ERR_HIP, "HIP error %d: %s", (int)e, hipGetErrorString(e));
}

fa_status fwd_impl(fa_dtype dtype, const void* q, fa_strides q_strides, const void* k,
                   fa_strides k_strides, const void* v, fa_strides v_strides, void* o,
                   fa_strides o_strides, float* lse, int B, int H, int N, int Nk, int d,
                   float scale, int causal, const int32_t* seqlens_k,
                   const uint8_t* block_mask, int mask_block, float dropout_p, uint64_t seed,
                   uint32_t offset, int block_q, hipStream_t stream) {
  int al = 0;
  fa_status st = check_common(dtype, B, H, N, Nk, d, scale, block_mask, mask_block, &al);
  if (st != FA_OK) return st;
  if ((st = check_tensor("q", q, q_strides, al, N)) != FA_OK) return st;
  if ((st = check_tensor("k", k, k_strides, al, Nk)) != FA_OK) return st;
  if ((st = check_tensor("v", v, v_strides, al, Nk)) != FA_OK) return st;
  if ((st = check_tensor("o", o, o_strides, al, N)) != FA_OK) return st;
  if (lse == nullptr) return fail(FA_ERR_INVALID_ARG, "lse is NULL");
  if (!aligned16(lse)) return fail(FA_ERR_INVALID_ARG, "lse is not 16-byte aligned");
  if (seqlens_k != nullptr && ((uintptr_t)seqlens_k & 3u))
    return fail(FA_ERR_INVALID_ARG, "seqlens_k is not 4-byte aligned");
  fa::Dropout drop{};
  if ((st = make_dropout(dropout_p, seed, offset, &drop)) != FA_OK) return st;
  if (block_q != 64 && block_q != 128 && block_q != 256)
    return fail(FA_ERR_INVALID_ARG, "block_q must be 64, 128 or 256 (got %d)", block_q);
  if (d != 64 && block_q != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dimension %d is built with block_q 128 only", d);
  if (drop.t < 256 && block_q != 128)
    return fail(FA_ERR_UNSUPPORTED, "dropout is built with block_q 128 only");
  if (block_q != 128 && dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "block_q other than 128 is built for bf16 only");
  if (block_mask != nullptr && mask_block % block_q != 0)
    return fail(FA_ERR_UNSUPPORTED, "block_q %d does not divide mask_block %d", block_q,
                mask_block);

  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.sq = cvt(q_strides);
  a.sk = cvt(k_strides);
  a.sv = cvt(v_strides);
  a.so = cvt(o_strides);
  a.B = B;
  a.H = H;
  a.N = N;
  a.Nk = Nk;
  a.coff = Nk - N;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.seqlens = seqlens_k;
  a.bmask = block_mask;
  a.mask_block = block_mask ? mask_block : 128;
  a.n_mask_q = (N + a.mask_block - 1) / a.mask_block;
  a.n_mask_k = (Nk + a.mask_block - 1) / a.mask_block;
  a.drop = drop;
  const hipError_t e = dtype == FA_BF16 ? fa::launch_fwd_bf16(a, causal != 0, block_q, d, stream)
                                        : fa::launch_fwd_f32(a, causal != 0, d, stream);
  return hip_status(e);
}

}  // namespace

extern "C" {

fa_status fa_fwd(fa_dtype dtype, const void* q, fa_strides q_strides, const void* k,
                 fa_strides k_strides, const void* v, fa_strides v_strides, void* o,
                 fa_strides o_strides, float* lse, int B, int H, int N, int d, float scale,
                 int causal, const int32_t* seqlens_k, const uint8_t* block_mask,
                 int mask_block, hipStream_t stream) {
  return fwd_impl(dtype, q, q_strides, k, k_strides, v, v_strides, o, o_strides, lse, B, H, N,
                  N, d, scale, causal, seqlens_k, block_mask, mask_block, 0.f, 0, 0, 128, stream);
}

fa_status fa_fwd_tiled(fa_dtype dtype, const void* q, fa_strides q_strides, const void* k,
                       fa_strides k_strides, const void* v, fa_strides v_strides, void* o,
                       fa_strides o_strides, float* lse, int B, int H, int N, int d, float scale,
                       int causal, const int32_t* seqlens_k, const uint8_t* block_mask,
                       int mask_block, int block_q, hipStream_t stream) {
  return fwd_impl(dtype, q, q_strides, k, k_strides, v, v_strides, o, o_strides, lse, B, H, N,
                  N, d, scale, causal, seqlens_k, block_mask, mask_block, 0.f, 0, 0, block_q,
                  stream);
}

fa_status fa_fwd_qk(fa_dtype dtype, const void* q, fa_strides q_strides, const void* k,
                    fa_strides k_strides, const void* v, fa_strides v_strides, void* o,
                    fa_strides o_strides, float* lse, int B, int H, int N_q, int N_k, int d,
                    float scale, int causal, const int32_t* seqlens_k,
                    const uint8_t* block_mask, int mask_block, float dropout_p, uint64_t seed,
                    uint32_t offset, hipStream_t stream) {
  return fwd_impl(dtype, q, q_strides, k, k_strides, v, v_strides, o, o_strides, lse, B, H, N_q,
                  N_k, d, scale, causal, seqlens_k, block_mask, mask_block, dropout_p, seed,
                  offset, 128, stream);
}

fa_status fa_fwd_dropout(fa_dtype dtype, const void* q, fa_strides q_strides, const void* k,
                         fa_strides k_strides, const void* v, fa_strides v_strides, void* o,
                         fa_strides o_strides, float* lse, int B, int H, int N, int d,
                         float scale, int causal, const int32_t* seqlens_k,
                         const uint8_t* block_mask, int mask_block, float dropout_p,
                         uint64_t seed, uint32_t offset, hipStream_t stream) {
  return fwd_impl(dtype, q, q_strides, k, k_strides, v, v_strides, o, o_strides, lse, B, H, N,
                  N, d, scale, causal, seqlens_k, block_mask, mask_block, dropout_p, seed, offset,
                  128, stream);
}

size_t fa_bwd_workspace_bytes(fa_dtype dtype, int B, int H, int N, int d) {
  // The bf16 backward pass writes D_i = dot(dO_i, O_i) of every query row to
  // the workspace before its main kernel; the fp32 kernels keep D on chip.
  (void)d;
  if (dtype != FA_BF16 || B <= 0 || H <= 0 || N <= 0) return 0;
  return fa::bwd_workspace_bytes(B, H, N);
}

int fa_fwd_key_groups(fa_dtype dtype, int B, int H, int N, int N_k, int d, int block_q) {
  if (dtype != FA_BF16 || B <= 0 || H <= 0 || N <= 0 || N_k <= 0) return 1;
  return fa::fwd_key_groups(B, H, N, N_k, d, block_q);
}

}  // extern "C"

namespace {

// Device memory of the allocation-free backward entry point (fa_bwd_noalloc):
// D of up to kScratchRows query rows.  Each GPU the library runs on holds its
// own copy of this array until the process ends.  Host code never uses the
// array's name as a device address (on the host it is only a stand-in): the
// address is read once per device with hipGetSymbolAddress and kept in
// g_scratch_ptr.
constexpr size_t kScratchRows = (size_t)1 << 22;
__device__ __align__(256) float scratch[kScratchRows];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The scratch array's address on the current device, read on the first call
// made with that device current.
fa_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FA_ERR_UNSUPPORTED, "device %d: fa_bwd_noalloc supports devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

// static_scratch: use the library's scratch array instead of the caller's
// workspace (whose arguments are then ignored); sizes beyond it are rejected
// before any HIP call.
fa_status bwd_impl(int phases, fa_dtype dtype, const void* q, fa_strides q_strides,
                   const void* k, fa_strides k_strides, const void* v, fa_strides v_strides,
                   const void* o, fa_strides o_strides, const void* dout,
                   fa_strides dout_strides, const float* lse, void* dq, fa_strides dq_strides,
                   void* dk, fa_strides dk_strides, void* dv, fa_strides dv_strides,
                   void* workspace, size_t workspace_bytes, int B, int H, int N, int Nk, int d,
                   float scale, int causal, const int32_t* seqlens_k,
                   const uint8_t* block_mask, int mask_block, float dropout_p, uint64_t seed,
                   uint32_t offset, hipStream_t stream, bool static_scratch = false) {
  int al = 0;
  fa_status st = check_common(dtype, B, H, N, Nk, d, scale, block_mask, mask_block, &al);
  if (st != FA_OK) return st;
  const size_t need = fa_bwd_workspace_bytes(dtype, B, H, N, d);
  if (static_scratch) {
    if (need > sizeof(scratch))
      return fail(FA_ERR_UNSUPPORTED,
                  "fa_bwd_noalloc: B * H * N = %lld query rows exceed its %zu-row scratch array",
                  (long long)B * H * N, kScratchRows);
    workspace = nullptr;
    workspace_bytes = need;
  }
  if ((st = check_tensor("q", q, q_strides, al, N)) != FA_OK) return st;
  if ((st = check_tensor("k", k, k_strides, al, Nk)) != FA_OK) return st;
  if ((st = check_tensor("v", v, v_strides, al, Nk)) != FA_OK) return st;
  if ((st = check_tensor("o", o, o_strides, al, N)) != FA_OK) return st;
  if (phases & fa::kPhaseDQ) {
    if ((st = check_tensor("dq", dq, dq_strides, al, N)) != FA_OK) return st;
  }
  if ((st = check_tensor("dout", dout, dout_strides, al, N)) != FA_OK) return st;
  if (phases & fa::kPhaseDKDV) {
    if ((st = check_tensor("dk", dk, dk_strides, al, Nk)) != FA_OK) return st;
    if ((st = check_tensor("dv", dv, dv_strides, al, Nk)) != FA_OK) return st;
  }
  if (lse == nullptr) return fail(FA_ERR_INVALID_ARG, "lse is NULL");
  if (!aligned16(lse)) return fail(FA_ERR_INVALID_ARG, "lse is not 16-byte aligned");
  if (need > 0 && !static_scratch) {
    if (workspace == nullptr) return fail(FA_ERR_INVALID_ARG, "workspace is NULL");
    if (!aligned16(workspace))
      return fail(FA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_INVALID_ARG, "workspace too small: %zu < %zu bytes", workspace_bytes,
                  need);
  }
  if (seqlens_k != nullptr && ((uintptr_t)seqlens_k & 3u))
    return fail(FA_ERR_INVALID_ARG, "seqlens_k is not 4-byte aligned");
  fa::Dropout drop{};
  if ((st = make_dropout(dropout_p, seed, offset, &drop)) != FA_OK) return st;
  if (static_scratch && need > 0) {  // every argument checked: the first HIP calls
    if ((st = scratch_address(&workspace)) != FA_OK) return st;
  }

  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dsum = need > 0 ? static_cast<float*>(workspace) : nullptr;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.sq = cvt(q_strides);
  a.sk = cvt(k_strides);
  a.sv = cvt(v_strides);
  a.so = cvt(o_strides);
  a.sdo = cvt(dout_strides);
  a.sdq = cvt(dq_strides);
  a.sdk = cvt(dk_strides);
  a.sdv = cvt(dv_strides);
  a.B = B;
  a.H = H;
  a.N = N;
  a.Nk = Nk;
  a.coff = Nk - N;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.seqlens = seqlens_k;
  a.bmask = block_mask;
  a.mask_block = block_mask ? mask_block : 128;
  a.n_mask_q = (N + a.mask_block - 1) / a.mask_block;
  a.n_mask_k = (Nk + a.mask_block - 1) / a.mask_block;
  a.drop = drop;
  const hipError_t e = dtype == FA_BF16 ? fa::launch_bwd_bf16(a, causal != 0, phases, d, stream)
                                        : fa::launch_bwd_f32(a, causal != 0, phases, d, stream);
  return hip_status(e);
}

}  // namespace

extern "C" {

fa_status fa_bwd(fa_dtype dtype, const void* q, fa_strides q_strides, const void* k,
                 fa_strides k_strides, const void* v, fa_strides v_strides, const void* o,
                 fa_strides o_strides, const void* dout, fa_strides dout_strides,
                 const float* lse, void* dq, fa_strides dq_strides, void* dk,
                 fa_strides dk_strides, void* dv, fa_strides dv_strides, void* workspace,
                 size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                 const int32_t* seqlens_k, const uint8_t* block_mask, int mask_block,
                 hipStream_t stream) {
  return bwd_impl(fa::kPhaseDQ | fa::kPhaseDKDV, dtype, q, q_strides, k, k_strides, v,
                  v_strides, o, o_strides, dout, dout_strides, lse, dq, dq_strides, dk,
                  dk_strides, dv, dv_strides, workspace, workspace_bytes, B, H, N, N, d, scale,
                  causal, seqlens_k, block_mask, mask_block, 0.f, 0, 0, stream);
}

fa_status fa_bwd_qk(fa_dtype dtype, const void* q, fa_strides q_strides, const void* k,
                    fa_strides k_strides, const void* v, fa_strides v_strides, const void* o,
                    fa_strides o_strides, const void* dout, fa_strides dout_strides,
                    const float* lse, void* dq, fa_strides dq_strides, void* dk,
                    fa_strides dk_strides, void* dv, fa_strides dv_strides, void* workspace,
                    size_t workspace_bytes, int B, int H, int N_q, int N_k, int d, float scale,
                    int causal, const int32_t* seqlens_k, const uint8_t* block_mask,
                    int mask_block, float dropout_p, uint64_t seed, uint32_t offset,
                    hipStream_t stream) {
  return bwd_impl(fa::kPhaseDQ | fa::kPhaseDKDV, dtype, q, q_strides, k, k_strides, v,
                  v_strides, o, o_strides, dout, dout_strides, lse, dq, dq_strides, dk,
                  dk_strides, dv, dv_strides, workspace, workspace_bytes, B, H, N_q, N_k, d,
                  scale, causal, seqlens_k, block_mask, mask_block, dropout_p, seed, offset,
                  stream);
}

fa_status fa_bwd_dropout(fa_dtype dtype, const void* q, fa_strides q_strides, const void* k,
                         fa_strides k_strides, const void* v, fa_strides v_strides,
                         const void* o, fa_strides o_strides, const void* dout,
                         fa_strides dout_strides, const float* lse, void* dq,
                         fa_strides dq_strides, void* dk, fa_strides dk_strides, void* dv,
                         fa_strides dv_strides, void* workspace, size_t workspace_bytes, int B,
                         int H, int N, int d, float scale, int causal,
                         const int32_t* seqlens_k, const uint8_t* block_mask, int mask_block,
                         float dropout_p, uint64_t seed, uint32_t offset, hipStream_t stream) {
  return bwd_impl(fa::kPhaseDQ | fa::kPhaseDKDV, dtype, q, q_strides, k, k_strides, v,
                  v_strides, o, o_strides, dout, dout_strides, lse, dq, dq_strides, dk,
                  dk_strides, dv, dv_strides, workspace, workspace_bytes, B, H, N, N, d, scale,
                  causal, seqlens_k, block_mask, mask_block, dropout_p, seed, offset, stream);
}

fa_status fa_bwd_noalloc(fa_dtype dtype, const void* q, fa_strides q_strides, const void* k,
                         fa_strides k_strides, const void* v, fa_strides v_strides,
                         const void* o, fa_strides o_strides, const void* dout,
                         fa_strides dout_strides, const float* lse, void* dq,
                         fa_strides dq_strides, void* dk, fa_strides dk_strides, void* dv,
                         fa_strides dv_strides, int B, int H, int N, int d, float scale,
                         int causal, const int32_t* seqlens_k, const uint8_t* block_mask,
                         int mask_block, hipStream_t stream) {
  return bwd_impl(fa::kPhaseDQ | fa::kPhaseDKDV, dtype, q, q_strides, k, k_strides, v,
                  v_strides, o, o_strides, dout, dout_strides, lse, dq, dq_strides, dk,
                  dk_strides, dv, dv_strides, nullptr, 0, B, H, N, N, d, scale, causal,
                  seqlens_k, block_mask, mask_block, 0.f, 0, 0, stream, true);
}

fa_status fa_bwd_dq(fa_dtype dtype, const void* q, fa_strides q_strides, const void* k,
                    fa_strides k_strides, const void* v, fa_strides v_strides, const void* o,
                    fa_strides o_strides, const void* dout, fa_strides dout_strides,
                    const float* lse, void* dq, fa_strides dq_strides, void* workspace,
                    size_t workspace_bytes, int B, int H, int N, int d, float scale,
                    int causal, const int32_t* seqlens_k, const uint8_t* block_mask,
                    int mask_block, hipStream_t stream) {
  const fa_strides none{0, 0, 0};
  return bwd_impl(fa::kPhaseDQ, dtype, q, q_strides, k, k_strides, v, v_strides, o,
                  o_strides, dout, dout_strides, lse, dq, dq_strides, nullptr, none, nullptr,
                  none, workspace, workspace_bytes, B, H, N, N, d, scale, causal, seqlens_k,
                  block_mask, mask_block, 0.f, 0, 0, stream);
}

fa_status fa_bwd_dkdv(fa_dtype dtype, const void* q, fa_strides q_strides, const void* k,
                      fa_strides k_strides, const void* v, fa_strides v_strides,
                      const void* o, fa_strides o_strides, const void* dout,
                      fa_strides dout_strides, const float* lse, void* dk,
                      fa_strides dk_strides, void* dv, fa_strides dv_strides, void* workspace,
                      size_t workspace_bytes, int B, int H, int N, int d, float scale,
                      int causal, const int32_t* seqlens_k, const uint8_t* block_mask,
                      int mask_block, hipStream_t stream) {
  const fa_strides none{0, 0, 0};
  return bwd_impl(fa::kPhaseDKDV, dtype, q, q_strides, k, k_strides, v, v_strides, o,
                  o_strides, dout, dout_strides, lse, nullptr, none, dk, dk_strides, dv,
                  dv_strides, workspace, workspace_bytes, B, H, N, N, d, scale, causal, seqlens_k,
                  block_mask, mask_block, 0.f, 0, 0, stream);
}

const char* fa_status_string(fa_status status) {
  switch (status) {
    case FA_OK:
      return "FA_OK";
    case FA_ERR_INVALID_ARG:
      return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP:
      return "FA_ERR_HIP";
  }
  return "FA_UNKNOWN_STATUS";
}

const char* fa_last_error(void) { return g_err; }

}  // extern "C"
