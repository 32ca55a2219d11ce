"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The GPU library never calls it and shares no code with it.

What it computes.  The FlashAttention pages claim an exact method: the output
equals standard attention, only computed with fewer HBM accesses
(researchpapers.dev explainer "FlashAttention 详解", sections "quick answer"
and FAQ "exact or approximate?"; suanlizi.com summary, closing paragraph of
"core idea").  So the oracle is standard attention written out with the
N x N probability matrix P materialised (suanlizi.com, "kernel fusion" and
"tiling": standard attention computes S and P in full), in float64, chunked by
query rows only to bound memory:

    s_ij = scale * q_i . k_j,   masked entries set to -inf
    m_i  = max_j s_ij,          P_ij = exp(s_ij - m_i) / sum_j exp(s_ij - m_i)
    O_i  = sum_j P_ij v_j,      L_i  = m_i + ln sum_j exp(s_ij - m_i)

The max subtraction is the "safe softmax" of the llm-deploy note
(flash-attention.md, overflow / underflow paragraphs).  The mask is the
intersection of: causal (key j visible to query i iff j <= i), key padding
(j < len_b) and a tile mask indexed [query tile][key tile] (suanlizi.com,
"block-sparse attention": only the important blocks are computed).

Backward.  The pages only say that the backward pass recomputes the attention
blocks from the saved softmax statistics (researchpapers.dev, "tiling and
recomputation"); the gradient formulas are not printed.  They follow from
differentiating the definitions above for f = sum(dO * O):

    dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
    dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q

Readings where the pages are silent (each also listed in the design notes):
rows with no visible key give O_i = 0, L_i = -inf and no gradient; keys past a
sequence's length get dK = dV = 0; L is the natural-log logsumexp.  The pages
only treat square problems; with N_q queries and N_k keys (the queries being
the last N_q positions of a sequence whose first N_k - N_q keys are already
cached), causal visibility is j <= i + (N_k - N_q), so the last query sees
every key, and the tile mask is [ceil(N_q / mb)][ceil(N_k / mb)].

Every function here is pinned by tests that do not re-use its formula:
closed forms, invariants, a hand-worked fixture, central finite differences,
an online-softmax evaluation and a library cross-check
(tests/test_oracle.py).
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 256


def visible(rows: np.ndarray, n_keys: int, causal: bool, seqlen, block_mask,
            mask_block: int, n_queries=None) -> np.ndarray:
    """bool ``[len(rows), n_keys]``: True where query ``rows[r]`` may attend key
    j.  ``n_queries`` (default n_keys) sets the causal offset N_k - N_q."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(n_keys, dtype=np.int64)
    off = 0 if n_queries is None else n_keys - n_queries
    vis = np.ones((rows.size, n_keys), dtype=bool)
    if causal:
        vis &= j[None, :] <= rows[:, None] + off
    if seqlen is not None:
        vis &= j[None, :] < int(seqlen)
    if block_mask is not None:
        bm = np.asarray(block_mask).astype(bool)
        vis &= bm[rows // mask_block][:, j // mask_block]
    return vis


def _probabilities(qr: np.ndarray, k: np.ndarray, vis: np.ndarray, scale: float):
    """Two-pass safe softmax of one row block: returns (P, L)."""
    s = scale * (qr @ k.T)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    dead = ~np.isfinite(m)
    m0 = np.where(dead, 0.0, m)
    e = np.exp(s - m0[:, None])
    l = e.sum(axis=1)
    l1 = np.where(dead, 1.0, l)
    p = e / l1[:, None]
    lse = np.where(dead, -np.inf, m0 + np.log(l1))
    return p, lse


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _rows_for(bh_rows, N):
    return np.arange(N, dtype=np.int64) if bh_rows is None else np.asarray(bh_rows, np.int64)


def forward(q, k, v, scale, causal=False, seqlens=None, block_mask=None,
            mask_block=128, rows=None):
    """Standard attention forward.

    q: ``[B, H, N_q, d]``; k, v: ``[B, H, N_k, d]`` (any float dtype;
    computed in float64).
    rows: None (all rows) or int ``[B, H, R]`` query rows to evaluate.
    Returns O ``[B, H, R, d]`` and L ``[B, H, R]`` (R = N_q when rows is None).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, _ = q.shape
    Nk = k.shape[2]
    dv = v.shape[-1]
    R = N if rows is None else rows.shape[-1]
    O = np.zeros((B, H, R, dv))
    L = np.zeros((B, H, R))
    for b in range(B):
        sl = None if seqlens is None else int(seqlens[b])
        for h in range(H):
            rr = _rows_for(None if rows is None else rows[b, h], N)
            for c0 in range(0, R, ROW_CHUNK):
                idx = rr[c0:c0 + ROW_CHUNK]
                vis = visible(idx, Nk, causal, sl, block_mask, mask_block, N)
                p, lse = _probabilities(q[b, h, idx], k[b, h], vis, scale)
                O[b, h, c0:c0 + idx.size] = p @ v[b, h]
                L[b, h, c0:c0 + idx.size] = lse
    return O, L


def backward(q, k, v, do, scale, causal=False, seqlens=None, block_mask=None,
             mask_block=128, rows=None):
    """Gradients of f = sum(dO * O) with respect to Q, K and V.

    rows None: full gradients dQ ``[B, H, N_q, d]``, dK, dV ``[B, H, N_k, d]``.
    rows ``[B, H, R]``: dQ ``[B, H, R, d]`` for those rows (exact full-problem
    values, since dQ_i depends on row i of dO only) and dK, dV ``[B, H, N_k, d]``
    of the restricted problem in which dO is zero outside the sampled rows.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, N, d = q.shape
    Nk = k.shape[2]
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
                p, _ = _probabilities(qc, kb, vis, scale)
                dV[b, h] += p.T @ doc
                dp = doc @ vb.T
                D = (p * dp).sum(axis=1)
                ds = p * (dp - D[:, None])
                dQ[b, h, c0:c0 + idx.size] = scale * (ds @ kb)
                dK[b, h] += scale * (ds.T @ qc)
    return dQ, dK, dV


def forward_online(q, k, v, scale, causal=False, seqlens=None, block_mask=None,
                   mask_block=128, key_block=64):
    """The pages' online softmax, taken literally on the CPU in float64.

    Keys are visited in blocks; each row keeps a running maximum m and a
    running sum l, and the partial output is rescaled whenever a new block
    raises the maximum (researchpapers.dev, "tiling and recomputation";
    llm-deploy note, the statistics (m, l) in its closing "solution" line).
    It never holds a full row of P.  Used only to pin that this procedure and
    the two-pass definition in ``forward`` agree.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, _ = q.shape
    Nk = k.shape[2]
    d = v.shape[-1]
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    rows = np.arange(N)
    for b in range(B):
        sl = None if seqlens is None else int(seqlens[b])
        for h in range(H):
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, d))
            for j0 in range(0, Nk, key_block):
                j1 = min(Nk, j0 + key_block)
                vis = visible(rows, Nk, causal, sl, block_mask, mask_block, N)[:, j0:j1]
                s = scale * (q[b, h] @ k[b, h, j0:j1].T)
                s = np.where(vis, s, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                live = np.isfinite(m_new)
                m_ref = np.where(live, m_new, 0.0)
                # rescale factor for what was accumulated under the old maximum
                alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
                p = np.exp(s - m_ref[:, None])
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, h, j0:j1]
                m = m_new
            dead = l == 0.0
            O[b, h] = np.where(dead[:, None], 0.0, acc / np.where(dead, 1.0, l)[:, None])
            L[b, h] = np.where(dead, -np.inf, m + np.log(np.where(dead, 1.0, l)))
    return O, L


def visible_pair_count(N, causal=False, seqlens=None, block_mask=None, mask_block=128,
                       B=1, N_k=None):
    """Brute-force count of visible (query, key) pairs summed over the batch
    (per head), by materialising the mask (N queries, N_k keys, default N)."""
    Nk = N if N_k is None else N_k
    total = 0
    for b in range(B):
        sl = None if seqlens is None else int(seqlens[b])
        total += int(visible(np.arange(N), Nk, causal, sl, block_mask, mask_block, N).sum())
    return total
