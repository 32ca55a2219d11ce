/*
 * fa.h -- C ABI of the exact, IO-aware, tiled attention library (libfa.so).
 *
 * The operation is exact softmax attention computed tile by tile without
 * ever storing the N x N score or probability matrix in device memory:
 *   suanlizi.com summary of FlashAttention, "tiling" and "kernel fusion"
 *     (Q, K, V are processed block by block inside one fused kernel);
 *   researchpapers.dev explainer "FlashAttention 详解", "tiling and
 *     recomputation" (online softmax with a running maximum and sum; the
 *     backward pass recomputes attention blocks from saved statistics);
 *   suanlizi.com, "block-sparse attention" (only kept blocks are computed).
 *
 * Definitions (per batch b, head h, query i, key j):
 *   s_ij = scale * dot(q_i, k_j)
 *   visible(i, j) = (!causal || j <= i) && (j < len_b) && block_mask[i/mb][j/mb]
 *   L_i  = ln sum_{visible j} exp(s_ij)      (natural-log logsumexp, fp32)
 *   O_i  = sum_{visible j} exp(s_ij - L_i) v_j
 * A row with no visible key gets O_i = 0 and L_i = -inf and contributes no
 * gradient.  The backward pass returns the gradients of sum(dO * O).
 *
 * Tensor layout.  Q, K, V, O, dO, dQ, dK, dV are rank-4 tensors indexed
 * [b][h][n][e] (e < d).  Each has its own fa_strides giving the element
 * strides of b, h and n; the e dimension must be contiguous (stride 1).  So
 * both [B,H,N,d] and [B,N,H,d] storage are accepted.  L (lse) is always a
 * contiguous fp32 [B,H,N] array.
 *
 * Ownership and synchronisation.  The caller owns every buffer (device
 * memory).  The library never allocates or frees memory, keeps no state
 * between calls apart from a per-thread error message, and is safe to call
 * from several host threads.  Work is enqueued on `stream` (NULL = the
 * default stream) and the call returns without synchronising; a device fault
 * surfaces at the caller's next synchronisation.  Outputs must not alias
 * inputs.  All argument checks run on the host before any HIP call, so a
 * rejected call touches no device state.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V, O, dO, dQ, dK, dV.  L and internal statistics are
 * always fp32. */
typedef enum fa_dtype {
  FA_BF16 = 0,
  FA_F32 = 1
} fa_dtype;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, bad size, stride or alignment, scale <= 0,
                             workspace too small, bad mask_block, bad dropout_p */
  FA_ERR_UNSUPPORTED = 2, /* valid request the library does not implement (d other than
                             32/64/128, too many mask tiles) */
  FA_ERR_HIP = 3          /* a HIP launch reported an error */
} fa_status;

/* Element strides of the batch, head and sequence dimensions. */
typedef struct fa_strides {
  int64_t batch;
  int64_t head;
  int64_t seq;
} fa_strides;

/*
 * fa_fwd -- forward pass: writes O and L.
 *
 *   dtype        FA_BF16 or FA_F32: element type of q, k, v and o.
 *   q, k, v      device pointers, [B][H][N][d] through their strides.
 *   o            device pointer, same element type, written in full.
 *   lse          device fp32 [B*H*N], contiguous, written in full (L above).
 *   B, H, N      >= 1.
 *   d            head dimension: 32, 64 or 128, either dtype, with or without
 *                dropout (FA_ERR_UNSUPPORTED otherwise).
 *   scale        score scale (> 0, finite), typically 1/sqrt(d).
 *   causal       nonzero: key j is visible to query i only if j <= i.
 *   seqlens_k    NULL, or device int32[B]: keys j >= seqlens_k[b] are masked
 *                (values are clamped to [0, N]).  Query rows are not masked.
 *   block_mask   NULL, or device uint8[T*T], T = ceil(N / mask_block), row-major
 *                [query tile][key tile], shared by all (b, h); nonzero = kept.
 *                Skipped tiles are never loaded or computed.
 *   mask_block   tile edge of block_mask, a positive multiple of 128 (ignored
 *                when block_mask is NULL).
 *   stream       HIP stream.
 * Alignment: every pointer 16-byte aligned; for bf16 every stride a multiple
 * of 8, for fp32 a multiple of 4.
 */
fa_status fa_fwd(fa_dtype dtype,
                 const void* q, fa_strides q_strides,
                 const void* k, fa_strides k_strides,
                 const void* v, fa_strides v_strides,
                 void* o, fa_strides o_strides,
                 float* lse,
                 int B, int H, int N, int d,
                 float scale, int causal,
                 const int32_t* seqlens_k,
                 const uint8_t* block_mask, int mask_block,
                 hipStream_t stream);

/*
 * fa_bwd_workspace_bytes -- device workspace that fa_bwd, fa_bwd_dq,
 * fa_bwd_dkdv, fa_bwd_dropout and fa_bwd_qk need.  The bf16 backward pass
 * first writes D_i = dot(dO_i, O_i) of every query row there (fp32, one
 * value per row; the quantity its gradient formula subtracts from dP, which
 * the pages leave to be derived -- researchpapers.dev explainer, "tiling and
 * recomputation": the backward pass recomputes from saved statistics), and
 * its main kernel reads it back.  Result: 4 * B * H * N bytes rounded up to
 * a multiple of 256 for FA_BF16 (N = the number of query rows, N_q for
 * fa_bwd_qk), 0 for FA_F32 (whose kernels keep D on chip) and for
 * non-positive sizes.  Linear in N: nothing of size N x N.  The contents on
 * return are D (callers may ignore them); they need no initialisation.
 */
size_t fa_bwd_workspace_bytes(fa_dtype dtype, int B, int H, int N, int d);

/*
 * fa_fwd_key_groups -- how many groups of waves a forward call with these
 * sizes splits each query tile's key range over, on the current device.  A
 * query tile is one workgroup; when the grid holds no more of them than the
 * device has CUs, each workgroup would run one wave per SIMD, so the bf16
 * forward with block_q = 128 and N_k >= 1024 keys gives each query tile 3
 * groups of 4 waves (2 for d = 128), each taking an equal run of the visible
 * key tiles with its own LDS buffers, and merges their partial results
 * (running maximum, sum and unnormalised output) with the online-softmax
 * rescaling (researchpapers.dev explainer, "tiling and recomputation").
 * The outputs are the same function of the inputs either way; only the
 * order of the floating-point sums differs.
 *
 *   dtype, B, H, N, N_k, d, block_q  as for fa_fwd_qk / fa_fwd_tiled
 *                                    (block_q = 128 for fa_fwd).
 * Returns the group count (1 = no split); it reads the device's CU count and
 * returns 1 if that fails.  No device memory is touched.
 */
int fa_fwd_key_groups(fa_dtype dtype, int B, int H, int N, int N_k, int d, int block_q);

/*
 * fa_bwd -- backward pass: writes dQ, dK and dV in full (zeros for keys that
 * no query sees, e.g. keys past seqlens_k).  The scores and probabilities are
 * recomputed tile by tile from q, k and the forward's lse; nothing of size
 * N x N is read or written.  Two kernel launches: the D pass, then one
 * kernel for all of dQ, dK and dV.
 *
 *   q, k, v, o, lse  the forward pass's inputs and outputs (o and lse as
 *                    written by fa_fwd with the same mask arguments).
 *   dout             upstream gradient dO, [B][H][N][d] through its strides.
 *   dq, dk, dv       outputs, element type dtype, through their strides.
 *   workspace        device buffer of at least fa_bwd_workspace_bytes(...) bytes
 *                    (16-byte aligned), overwritten; may be NULL only when that
 *                    size is 0 (FA_ERR_INVALID_ARG otherwise).  Two backward
 *                    calls that run at the same time need separate workspaces.
 *   remaining arguments as for fa_fwd and must match the forward call.
 */
fa_status fa_bwd(fa_dtype dtype,
                 const void* q, fa_strides q_strides,
                 const void* k, fa_strides k_strides,
                 const void* v, fa_strides v_strides,
                 const void* o, fa_strides o_strides,
                 const void* dout, fa_strides dout_strides,
                 const float* lse,
                 void* dq, fa_strides dq_strides,
                 void* dk, fa_strides dk_strides,
                 void* dv, fa_strides dv_strides,
                 void* workspace, size_t workspace_bytes,
                 int B, int H, int N, int d,
                 float scale, int causal,
                 const int32_t* seqlens_k,
                 const uint8_t* block_mask, int mask_block,
                 hipStream_t stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same two kernels and results as fa_bwd, but D lives in a
 * scratch array inside the library instead of a caller workspace, so there
 * are no workspace arguments.  The call itself allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).
 *
 *   arguments    as for fa_bwd, without workspace and workspace_bytes.
 *   limit        B * H * N <= 4194304 query rows for FA_BF16 (the array holds
 *                16 MiB of fp32 D); larger problems return FA_ERR_UNSUPPORTED
 *                before any HIP call.  FA_F32 needs no scratch.
 *   memory       each GPU the library runs on holds its own copy of the array
 *                (16 MiB) until the process ends; its device address is read
 *                once per device, on the first call made with that device
 *                current.
 *   concurrency  every call on one GPU shares that GPU's array, whose contents
 *                are the last call's D: two calls that overlap in time on one
 *                GPU (different streams, or different host threads without
 *                ordering) race and give wrong gradients.  Calls ordered on
 *                one stream are safe.  Nothing in the array has to start at
 *                zero (every row a call reads is written by that call first).
 */
fa_status fa_bwd_noalloc(fa_dtype dtype,
                         const void* q, fa_strides q_strides,
                         const void* k, fa_strides k_strides,
                         const void* v, fa_strides v_strides,
                         const void* o, fa_strides o_strides,
                         const void* dout, fa_strides dout_strides,
                         const float* lse,
                         void* dq, fa_strides dq_strides,
                         void* dk, fa_strides dk_strides,
                         void* dv, fa_strides dv_strides,
                         int B, int H, int N, int d,
                         float scale, int causal,
                         const int32_t* seqlens_k,
                         const uint8_t* block_mask, int mask_block,
                         hipStream_t stream);

/*
 * fa_bwd_dq, fa_bwd_dkdv -- the two halves of fa_bwd, each one kernel launch
 * of its own: fa_bwd_dq writes dQ, fa_bwd_dkdv writes dK and dV.  They are
 * independent of each other (either may run alone, in any order or on
 * different streams) and together give exactly what fa_bwd gives.  Both
 * read q, k, v, o, dout and lse; arguments mean what they mean for fa_bwd,
 * and validation and errors are the same.
 */
fa_status fa_bwd_dq(fa_dtype dtype,
                    const void* q, fa_strides q_strides,
                    const void* k, fa_strides k_strides,
                    const void* v, fa_strides v_strides,
                    const void* o, fa_strides o_strides,
                    const void* dout, fa_strides dout_strides,
                    const float* lse,
                    void* dq, fa_strides dq_strides,
                    void* workspace, size_t workspace_bytes,
                    int B, int H, int N, int d,
                    float scale, int causal,
                    const int32_t* seqlens_k,
                    const uint8_t* block_mask, int mask_block,
                    hipStream_t stream);

fa_status fa_bwd_dkdv(fa_dtype dtype,
                      const void* q, fa_strides q_strides,
                      const void* k, fa_strides k_strides,
                      const void* v, fa_strides v_strides,
                      const void* o, fa_strides o_strides,
                      const void* dout, fa_strides dout_strides,
                      const float* lse,
                      void* dk, fa_strides dk_strides,
                      void* dv, fa_strides dv_strides,
                      void* workspace, size_t workspace_bytes,
                      int B, int H, int N, int d,
                      float scale, int causal,
                      const int32_t* seqlens_k,
                      const uint8_t* block_mask, int mask_block,
                      hipStream_t stream);

/*
 * fa_fwd_tiled -- fa_fwd with a chosen query-tile height (bf16 only): each
 * workgroup owns block_q query rows (block_q / 32 waves) and streams the
 * visible K/V tiles of its (b, h) once, so the K/V bytes read from memory
 * scale like N^2 d / block_q.  This is the tile-size dependence of the pages'
 * IO analysis (researchpapers.dev explainer, "tiling and recomputation":
 * the on-chip tile bounds how often K and V are re-read), exposed for
 * measurement; fa_fwd uses 128.  Results equal fa_fwd's up to summation
 * order (block_q = 128 is the same kernel, bit for bit).
 *
 *   block_q      64, 128 or 256 (FA_ERR_INVALID_ARG otherwise).  With a
 *                block mask it must divide mask_block (FA_ERR_UNSUPPORTED).
 *                FA_F32 supports only 128 (FA_ERR_UNSUPPORTED).
 *   remaining arguments, validation and errors as for fa_fwd.
 */
fa_status fa_fwd_tiled(fa_dtype dtype,
                       const void* q, fa_strides q_strides,
                       const void* k, fa_strides k_strides,
                       const void* v, fa_strides v_strides,
                       void* o, fa_strides o_strides,
                       float* lse,
                       int B, int H, int N, int d,
                       float scale, int causal,
                       const int32_t* seqlens_k,
                       const uint8_t* block_mask, int mask_block,
                       int block_q,
                       hipStream_t stream);

/*
 * fa_fwd_dropout, fa_bwd_dropout -- fa_fwd and fa_bwd with dropout applied
 * to the probabilities.  The pages list dropout among the element-wise
 * operations that standard attention runs as separate kernels and that the
 * fused kernel absorbs (suanlizi.com summary, per-component timing figure of
 * "kernel fusion"); they give no formula, so the definition is:
 *
 *   O_i = sum_{visible j} s Z_ij exp(s_ij - L_i) v_j,   L_i as for fa_fwd
 *
 * (L stays the logsumexp of the undropped scores), with keep indicator Z_ij
 * and keep scale s = 256 / t, where t = floor(256 (1 - dropout_p) + 1/2)
 * computed in double.  Z_ij = 1 iff u_ij < t, u_ij being the pair's 8-bit
 * uniform number from Philox4x32 with 10 rounds (Salmon, Moraes, Dror and
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11) keyed by
 * (seed & 0xffffffff, seed >> 32): the call with counter
 * (j / 4, i / 4, b * H + h, offset) yields four 32-bit words, and u_ij is
 * byte j % 4 (least significant first) of word i % 4.  The effective drop
 * probability is therefore 1 - t / 256.  fa_bwd_dropout returns the
 * gradients of sum(dO * O) with the mask held fixed, and needs the same
 * dropout_p, seed and offset as the forward call (the mask is regenerated,
 * never stored).
 *
 *   dropout_p    in [0, 1); 0 gives exactly fa_fwd / fa_bwd.  A value that
 *                rounds to t = 0 is rejected (FA_ERR_INVALID_ARG).
 *   seed         64-bit Philox key.
 *   offset       fourth counter word: distinct offsets give independent
 *                masks under one seed.
 *   remaining arguments, validation and errors as for fa_fwd / fa_bwd.
 */
fa_status fa_fwd_dropout(fa_dtype dtype,
                         const void* q, fa_strides q_strides,
                         const void* k, fa_strides k_strides,
                         const void* v, fa_strides v_strides,
                         void* o, fa_strides o_strides,
                         float* lse,
                         int B, int H, int N, int d,
                         float scale, int causal,
                         const int32_t* seqlens_k,
                         const uint8_t* block_mask, int mask_block,
                         float dropout_p, uint64_t seed, uint32_t offset,
                         hipStream_t stream);

fa_status fa_bwd_dropout(fa_dtype dtype,
                         const void* q, fa_strides q_strides,
                         const void* k, fa_strides k_strides,
                         const void* v, fa_strides v_strides,
                         const void* o, fa_strides o_strides,
                         const void* dout, fa_strides dout_strides,
                         const float* lse,
                         void* dq, fa_strides dq_strides,
                         void* dk, fa_strides dk_strides,
                         void* dv, fa_strides dv_strides,
                         void* workspace, size_t workspace_bytes,
                         int B, int H, int N, int d,
                         float scale, int causal,
                         const int32_t* seqlens_k,
                         const uint8_t* block_mask, int mask_block,
                         float dropout_p, uint64_t seed, uint32_t offset,
                         hipStream_t stream);

/*
 * fa_fwd_qk, fa_bwd_qk -- the general forms: N_q queries attend to N_k keys
 * (every other entry point is the special case N_q = N_k, and fa_fwd /
 * fa_bwd also dropout_p = 0).  The pages only treat square problems; the
 * queries are read as the last N_q positions of a sequence whose first
 * N_k - N_q keys are already held (a key/value cache), so
 *
 *   causal: key j is visible to query i iff j <= i + (N_k - N_q)
 *
 * -- the last query sees every key, a single query (N_q = 1) sees all of
 * them, and with N_q > N_k the first N_q - N_k queries see none (O = 0,
 * L = -inf).  With N_q = N_k this is j <= i.
 *
 *   q, o, dout, dq   [B][H][N_q][d] through their strides; lse [B*H*N_q].
 *   k, v, dk, dv     [B][H][N_k][d] through their strides.
 *   seqlens_k        as before, clamped to [0, N_k].
 *   block_mask       uint8[ceil(N_q / mask_block) * ceil(N_k / mask_block)],
 *                    row-major [query tile][key tile].
 *   dropout_p, seed, offset  as for fa_fwd_dropout (0 = no dropout).
 *   remaining arguments, validation and errors as for fa_fwd / fa_bwd; N_k
 *   must be positive.
 */
fa_status fa_fwd_qk(fa_dtype dtype,
                    const void* q, fa_strides q_strides,
                    const void* k, fa_strides k_strides,
                    const void* v, fa_strides v_strides,
                    void* o, fa_strides o_strides,
                    float* lse,
                    int B, int H, int N_q, int N_k, int d,
                    float scale, int causal,
                    const int32_t* seqlens_k,
                    const uint8_t* block_mask, int mask_block,
                    float dropout_p, uint64_t seed, uint32_t offset,
                    hipStream_t stream);

fa_status fa_bwd_qk(fa_dtype dtype,
                    const void* q, fa_strides q_strides,
                    const void* k, fa_strides k_strides,
                    const void* v, fa_strides v_strides,
                    const void* o, fa_strides o_strides,
                    const void* dout, fa_strides dout_strides,
                    const float* lse,
                    void* dq, fa_strides dq_strides,
                    void* dk, fa_strides dk_strides,
                    void* dv, fa_strides dv_strides,
                    void* workspace, size_t workspace_bytes,
                    int B, int H, int N_q, int N_k, int d,
                    float scale, int causal,
                    const int32_t* seqlens_k,
                    const uint8_t* block_mask, int mask_block,
                    float dropout_p, uint64_t seed, uint32_t offset,
                    hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* fa_status_string(fa_status status);

/* Message describing the most recent failure on the calling thread (empty
 * string if none).  Valid until the next call on the same thread. */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
