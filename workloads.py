"""Seeded synthetic inputs for exact tiled attention.

This module only draws random numbers and rounds them to the storage format;
it holds none of the attention arithmetic.  Both the fp64 oracle tests and the
GPU path (tests, bench) take their inputs from here, so the two sides see
bit-identical operands.

Workloads are shaped after the models the FlashAttention pages train (GPT-2 at
1K, BERT-large at 512, long sequences up to 16K and block-sparse up to 64K;
suanlizi.com page, "core idea"; researchpapers.dev page, "key results").  No
dataset item is used: every tensor is iid Gaussian noise.

Draw order for one workload (one ``numpy.random.default_rng(seed)``, PCG64):
Q, K, V, dO (each ``[B, H, N, d]``, fp32 standard normals times ``std``; K and
V have ``N_k`` rows where a workload sets a key length of its own), then the
per-sequence key lengths or the tile mask, then the sampled query rows.
bf16 workloads round every tensor to bf16 with round-to-nearest-even and keep
it as float32 values that are exactly representable in bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

MASK_BLOCK = 128


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                 # "bf16" or "f32"
    causal: bool
    scale: float
    seed: int
    std: float = 1.0
    padded_min: Optional[int] = None   # key lengths uniform in [padded_min, N]
    block_keep_p: Optional[float] = None  # off-diagonal 128x128 tile keep probability
    sample_rows: Optional[int] = None  # query rows per (b, h) checked against the oracle
    backward: bool = True
    summary: str = field(default="", compare=False)
    Nk: Optional[int] = None   # keys, when not N (the queries are the last N positions)

    @property
    def n_keys(self) -> int:
        return self.N if self.Nk is None else self.Nk


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_f32_n128", 1, 1, 128, 64, "f32", False, 1 / 8, 1,
                 backward=False,
                 summary="single head, fp32, N=128, d=64, no mask, forward only"),
        Workload("gpt2s_causal_b8h12n1024", 8, 12, 1024, 64, "bf16", True, 1 / 8, 2,
                 summary="GPT-2-small shaped causal attention, bf16"),
        Workload("bertl_padded_b16h16n512", 16, 16, 512, 64, "bf16", False, 1 / 8, 3,
                 padded_min=256,
                 summary="BERT-large shaped attention, key padding, bf16"),
        Workload("long_causal_b1h16n16384", 1, 16, 16384, 64, "bf16", True, 1 / 8, 4,
                 std=0.5, sample_rows=1024,
                 summary="long-sequence causal attention, bf16"),
        Workload("blocksparse_b1h8n65536", 1, 8, 65536, 64, "bf16", False, 1 / 8, 5,
                 block_keep_p=1 / 16, sample_rows=512,
                 summary="block-sparse attention, 128x128 tiles, bf16"),
        Workload("causal_b2h32n4096d128", 2, 32, 4096, 128, "bf16", True, 128 ** -0.5, 8,
                 sample_rows=256, backward=False,
                 summary="7B-model-like causal attention, head dimension 128, bf16, forward"),
        Workload("train_causal_b2h16n4096d128", 2, 16, 4096, 128, "bf16", True, 128 ** -0.5, 9,
                 sample_rows=256,
                 summary="causal attention with head dimension 128, forward and backward, bf16"),
        Workload("train_causal_f32_b2h16n4096d128", 2, 16, 4096, 128, "f32", True,
                 128 ** -0.5, 10, sample_rows=256,
                 summary="causal attention with head dimension 128, forward and backward, "
                         "fp32"),
        Workload("prefill_causal_b1h16q2048k16384", 1, 16, 2048, 64, "bf16", True, 1 / 8, 7,
                 std=0.5, sample_rows=512, Nk=16384,
                 summary="chunked prefill: 2048 new queries over 16384 keys (14336 cached), "
                         "causal aligned to the last query, bf16"),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    bf16 keeps the top 16 bits of an IEEE binary32.  Adding 0x7FFF plus the
    lowest kept bit before truncating implements round-half-to-even.  Inputs
    here are finite Gaussian draws, so NaN/Inf handling is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    r = ((u + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The uint16 bf16 encoding of float32 values that are already bf16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-representable; round them first")
    return (u >> np.uint32(16)).astype(np.uint16)


def n_mask_tiles(N: int, mask_block: int = MASK_BLOCK) -> int:
    return (N + mask_block - 1) // mask_block


def draw_block_mask(rng: np.random.Generator, N: int, p: float,
                    mask_block: int = MASK_BLOCK) -> np.ndarray:
    """uint8 ``[T, T]`` tile mask, ``T = ceil(N / mask_block)``: the diagonal is
    always kept, every ordered off-diagonal pair independently with prob. p."""
    t = n_mask_tiles(N, mask_block)
    m = rng.random((t, t)) < p
    np.fill_diagonal(m, True)
    return m.astype(np.uint8)


def draw_tensors(rng: np.random.Generator, B: int, H: int, N: int, d: int,
                 dtype: str, std: float = 1.0, count: int = 4):
    out = []
    for _ in range(count):
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if std != 1.0:
            x = (x * np.float32(std)).astype(np.float32)
        if dtype == "bf16":
            x = round_to_bf16(x)
        out.append(x)
    return out


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """All inputs of one workload, drawn in the documented order."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if w.Nk is None:
        q, k, v, do = draw_tensors(rng, w.B, w.H, w.N, w.d, w.dtype, w.std)
    else:
        (q,) = draw_tensors(rng, w.B, w.H, w.N, w.d, w.dtype, w.std, count=1)
        k, v = draw_tensors(rng, w.B, w.H, w.Nk, w.d, w.dtype, w.std, count=2)
        (do,) = draw_tensors(rng, w.B, w.H, w.N, w.d, w.dtype, w.std, count=1)
    seqlens = None
    block_mask = None
    if w.padded_min is not None:
        seqlens = rng.integers(w.padded_min, w.N + 1, size=w.B).astype(np.int32)
    if w.block_keep_p is not None:
        block_mask = draw_block_mask(rng, w.N, w.block_keep_p)
    rows = None
    if w.sample_rows is not None:
        rows = sample_rows(rng, w.B, w.H, w.N, w.sample_rows)
    return dict(q=q, k=k, v=v, do=do, seqlens=seqlens, block_mask=block_mask,
                rows=rows, scale=w.scale, causal=w.causal, dtype=w.dtype)


def sample_rows(rng: np.random.Generator, B: int, H: int, N: int, R: int) -> np.ndarray:
    """``int64 [B, H, R]``: per (b, h) an independent sorted sample of R query
    rows drawn without replacement."""
    rows = np.empty((B, H, R), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            rows[b, h] = np.sort(rng.choice(N, size=R, replace=False))
    return rows


def random_case(B: int, H: int, N: int, d: int, *, dtype: str = "bf16", seed: int = 0,
                std: float = 1.0, causal: bool = False, seqlens=None,
                block_keep_p: Optional[float] = None, mask_block: int = MASK_BLOCK,
                scale: Optional[float] = None) -> dict:
    """A small seeded case for parity sweeps.  ``seqlens`` may be an explicit
    list, ``"random"`` (uniform in [0, N]) or None."""
    rng = np.random.default_rng(seed)
    q, k, v, do = draw_tensors(rng, B, H, N, d, dtype, std)
    if isinstance(seqlens, str) and seqlens == "random":
        seqlens = rng.integers(0, N + 1, size=B).astype(np.int32)
    elif seqlens is not None:
        seqlens = np.asarray(seqlens, dtype=np.int32)
    block_mask = None
    if block_keep_p is not None:
        block_mask = draw_block_mask(rng, N, block_keep_p, mask_block)
    return dict(q=q, k=k, v=v, do=do, seqlens=seqlens, block_mask=block_mask, rows=None,
                scale=(1.0 / np.sqrt(d)) if scale is None else scale, causal=causal,
                dtype=dtype, mask_block=mask_block)
