// Internal launch arguments shared by the host API (fa_api.hip) and the
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Key or query rows per LDS tile and per mask expansion unit.
constexpr int kTile = 64;
// Largest number of 64-row tiles a block-mask list may hold (N <= 262144).
constexpr int kMaxListTiles = 4096;

struct Strides {
  int64_t b, h, s;
};

// Dropout on the probabilities: a pair is kept iff its Philox byte is below
// t, and kept probabilities are multiplied by scale = 256 / t.  t = 256 keeps
// every pair (no dropout).
struct Dropout {
  uint32_t t;
  float scale;
  uint32_t seed_lo, seed_hi;
  uint32_t offset;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  Strides sq, sk, sv, so;
  int B, H;
  int N;     // queries
  int Nk;    // keys
  int coff;  // causal offset Nk - N: key j is visible to query i iff j <= i + coff
             // (the bf16 forward runs non-causal calls with coff = Nk)
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e): scores enter exp2 directly
  const int32_t* seqlens;
  const uint8_t* bmask;  // [n_mask_q][n_mask_k]
  int mask_block;
  int n_mask_q, n_mask_k;
  Dropout drop;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* dsum;  // D_i = dot(dO_i, O_i), fp32 [B*H*N] (the caller's workspace)
  void* dq;
  void* dk;
  void* dv;
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  int B, H;
  int N;     // queries (Q, O, dO, dQ, L rows)
  int Nk;    // keys (K, V, dK, dV rows)
  int coff;  // causal offset Nk - N
  float scale;
  float scale_log2;
  const int32_t* seqlens;
  const uint8_t* bmask;  // [n_mask_q][n_mask_k]
  int mask_block;
  int n_mask_q, n_mask_k;
  Dropout drop;
};

// Backward roles: kPhaseDQ writes dQ, kPhaseDKDV writes dK and dV.  They are
// independent; the full backward pass runs both in one launch.
constexpr int kPhaseDQ = 1;
constexpr int kPhaseDKDV = 2;

// block_q: query rows per workgroup, 64, 128 or 256 (128 with dropout);
// d: head dimension, 32, 64 or 128 (64 when block_q != 128).
hipError_t launch_fwd_bf16(const FwdArgs& a, bool causal, int block_q, int d,
                           hipStream_t stream);
// Wave groups per query tile that launch_fwd_bf16 splits the key range over
// on the current device: 3 (2 for d = 128) when block_q is 128, the keys span
// at least 1024 rows and the grid holds at most one query tile per CU, else 1.
int fwd_key_groups(int B, int H, int N, int Nk, int d, int block_q);
// Bytes of the bf16 backward's workspace: D for every query row.
inline size_t bwd_workspace_bytes(int B, int H, int N) {
  return (((size_t)B * H * N * 4) + 255) & ~(size_t)255;
}
// d: head dimension, 32, 64 or 128.  a.dsum must hold
// bwd_workspace_bytes(B, H, N) bytes.
hipError_t launch_bwd_bf16(const BwdArgs& a, bool causal, int phases, int d,
                           hipStream_t stream);
// The d = 128 instantiation of the above, from its own translation unit.
hipError_t launch_bwd_bf16_d128(const BwdArgs& a, bool causal, int phases,
                                hipStream_t stream);
// The fp32 kernels: 128 query (key) rows per workgroup, d = 32, 64 or 128
// (hipErrorInvalidValue otherwise); no workspace, each kernel forms D itself.
hipError_t launch_fwd_f32(const FwdArgs& a, bool causal, int d, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdArgs& a, bool causal, int phases, int d, hipStream_t stream);

}  // namespace fa
