"""fp64 CPU oracle for attention with dropout on P -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The GPU library never calls it and shares no code with it.

The pages list dropout among the element-wise operations that standard
attention runs as separate memory-bound kernels and that the fused kernel
absorbs (suanlizi.com summary, the per-component timing figure of "kernel
fusion"; researchpapers.dev explainer, the list of element-wise operations in
"why attention is memory-bound").  They print no formula, random number
generator or threshold, so everything below is a reading of that one
statement (each item is also in the design notes):

* Dropout acts on the normalised probabilities: with a keep indicator Z_ij
  and keep scale s,
      O_i = sum_j (s Z_ij P_ij) v_j,   L_i unchanged (the statistics of the
  undropped softmax, which is what the backward pass recomputes P from).
* Z_ij comes from a counter-based generator, so that the forward and the
  backward pass (and this oracle) regenerate the same mask without storing
  it: Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel
  random numbers: as easy as 1, 2, 3", SC'11, the Philox family), keyed by a
  64-bit seed (low word first).  One call covers a 4 x 4 block of (query,
  key) pairs:
      counter = (j div 4, i div 4, b H + h, offset),
      word (i mod 4) of the output, byte (j mod 4) of that word (byte 0 = the
      least significant) is the pair's 8-bit uniform number u_ij.
* Keep iff u_ij < t with t = floor(256 (1 - p) + 1/2); the effective drop
  probability is 1 - t / 256 and the keep scale is s = 256 / t, so that
  E[s Z] = 1 exactly.  p = 0 gives t = 256: every pair is kept, s = 1 and
  the result is plain attention.

Backward (calculus on the definition above, for f = sum(dO * O)):
    dV = (s Z P)^T dO,  dP = s Z (dO V^T),  D_i = sum_j P_ij dP_ij = dO_i . O_i,
    dS = P (dP - D),    dQ = scale dS K,     dK = scale dS^T Q.
"""
from __future__ import annotations

import numpy as np

from .attention_ref import ROW_CHUNK, _as64, _probabilities, _rows_for, visible

# Philox4x32 constants (SC'11, the Philox-4x32 parameters): the two round
# multipliers and the two Weyl increments added to the key between rounds.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32(counter, key, rounds: int = 10):
    """Philox4x32-R on arrays.

    counter: uint32-convertible array ``[..., 4]``; key: ``[..., 2]``
    (broadcast against counter).  Returns uint32 ``[..., 4]``.

    One round maps (x0, x1, x2, x3) with key (k0, k1) to
        (hi(M1 x2) ^ x1 ^ k0,  lo(M1 x2),  hi(M0 x0) ^ x3 ^ k1,  lo(M0 x0))
    where hi / lo are the upper / lower 32 bits of the 64-bit product; the
    key is advanced by (W0, W1) modulo 2^32 before every round after the
    first.
    """
    c = np.asarray(counter, dtype=np.uint64) & MASK32
    kk = np.asarray(key, dtype=np.uint64) & MASK32
    x0, x1, x2, x3 = (c[..., n] for n in range(4))
    k0 = np.broadcast_to(kk[..., 0], x0.shape).copy()
    k1 = np.broadcast_to(kk[..., 1], x0.shape).copy()
    m32 = np.uint64(MASK32)
    s32 = np.uint64(32)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & m32
            k1 = (k1 + np.uint64(PHILOX_W1)) & m32
        p0 = np.uint64(PHILOX_M0) * x0  # < 2^64: exact in uint64
        p1 = np.uint64(PHILOX_M1) * x2
        x0, x1, x2, x3 = ((p1 >> s32) ^ x1 ^ k0, p1 & m32, (p0 >> s32) ^ x3 ^ k1, p0 & m32)
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def keep_threshold(p: float) -> int:
    """t such that a pair is kept iff its 8-bit uniform number is below t."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    t = int(np.floor(256.0 * (1.0 - p) + 0.5))
    if t < 1:
        raise ValueError("dropout probability rounds to dropping every pair")
    return t


def uniform_bytes(rows, n_keys: int, bh: int, seed: int, offset: int) -> np.ndarray:
    """uint8 ``[len(rows), n_keys]``: u_ij of query rows ``rows`` of head
    slice ``bh`` for keys 0..n_keys-1."""
    rows = np.asarray(rows, dtype=np.int64)
    nb = (n_keys + 3) // 4
    ctr = np.zeros((rows.size, nb, 4), dtype=np.uint64)
    ctr[..., 0] = np.arange(nb, dtype=np.uint64)[None, :]
    ctr[..., 1] = (rows // 4).astype(np.uint64)[:, None]
    ctr[..., 2] = bh
    ctr[..., 3] = offset & MASK32
    key = np.array([seed & MASK32, (seed >> 32) & MASK32], dtype=np.uint64)
    words = philox4x32(ctr, key)                                   # [R, nb, 4]
    w = np.take_along_axis(words, (rows % 4)[:, None, None], axis=2)[..., 0]  # [R, nb]
    by = (w[..., None] >> (8 * np.arange(4, dtype=np.uint32))) & 0xFF  # [R, nb, 4]
    return by.reshape(rows.size, 4 * nb)[:, :n_keys].astype(np.uint8)


def keep_mask(rows, n_keys: int, bh: int, p: float, seed: int, offset: int) -> np.ndarray:
    """bool ``[len(rows), n_keys]``: Z_ij for the given rows of slice bh."""
    return uniform_bytes(rows, n_keys, bh, seed, offset) < keep_threshold(p)


def forward(q, k, v, scale, p, seed, offset=0, causal=False, seqlens=None, block_mask=None,
            mask_block=128, rows=None, n_heads=None):
    """Attention forward with dropout on P.  Shapes as in
    ``attention_ref.forward``; returns O and L (L of the undropped softmax).
    ``n_heads``: the head count that the mask index b H + h uses (default:
    the tensors' own; larger when the tensors are the first heads of a
    problem)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, _ = q.shape
    Nk = k.shape[2]
    Hm = H if n_heads is None else n_heads
    s = 256.0 / keep_threshold(p)
    R = N if rows is None else rows.shape[-1]
    O = np.zeros((B, H, R, v.shape[-1]))
    L = np.zeros((B, H, R))
    for b in range(B):
        sl = None if seqlens is None else int(seqlens[b])
        for h in range(H):
            rr = _rows_for(None if rows is None else rows[b, h], N)
            for c0 in range(0, R, ROW_CHUNK):
                idx = rr[c0:c0 + ROW_CHUNK]
                vis = visible(idx, Nk, causal, sl, block_mask, mask_block, N)
                pr, lse = _probabilities(q[b, h, idx], k[b, h], vis, scale)
                z = keep_mask(idx, Nk, b * Hm + h, p, seed, offset)
                O[b, h, c0:c0 + idx.size] = (s * z * pr) @ v[b, h]
                L[b, h, c0:c0 + idx.size] = lse
    return O, L


def backward(q, k, v, do, scale, p, seed, offset=0, causal=False, seqlens=None,
             block_mask=None, mask_block=128, rows=None, n_heads=None):
    """Gradients of f = sum(dO * O) for attention with dropout (the mask held
    fixed).  ``rows`` as in ``attention_ref.backward``: dQ of the sampled rows,
    dK and dV of the problem with dO zero outside them."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    Hm = H if n_heads is None else n_heads
    s = 256.0 / keep_threshold(p)
    R = N if rows is None else rows.shape[-1]
    dQ = np.zeros((B, H, R, d))
    dK = np.zeros((B, H, Nk, d))
    dV = np.zeros((B, H, Nk, v.shape[-1]))
    for b in range(B):
        sl = None if seqlens is None else int(seqlens[b])
        for h in range(H):
            rr = _rows_for(None if rows is None else rows[b, h], N)
            kb, vb = k[b, h], v[b, h]
            for c0 in range(0, R, ROW_CHUNK):
                idx = rr[c0:c0 + ROW_CHUNK]
                vis = visible(idx, Nk, causal, sl, block_mask, mask_block, N)
                qc, doc = q[b, h, idx], do[b, h, idx]
                pr, _ = _probabilities(qc, kb, vis, scale)
                sz = s * keep_mask(idx, Nk, b * Hm + h, p, seed, offset)
                dV[b, h] += (sz * pr).T @ doc
                dp = sz * (doc @ vb.T)
                D = (pr * dp).sum(axis=1)
                ds = pr * (dp - D[:, None])
                dQ[b, h, c0:c0 + idx.size] = scale * (ds @ kb)
                dK[b, h] += scale * (ds.T @ qc)
    return dQ, dK, dV
