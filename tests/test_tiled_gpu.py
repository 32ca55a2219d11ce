"""GPU parity of fa_fwd_tiled: the forward with 64- and 256-row query tiles
(2 and 8 waves per workgroup) against the fp64 oracle, and bit-identity of
the 128-row tile with fa_fwd (the same kernel)."""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import attention_ref as ref
from tests.gpu_util import TOL, device_inputs, maxabs, oracle_args, to_np

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(case, block_q):
    import torch
    import exact_io_aware_64_amd as fa
    q, k, v, _, sl, bm = device_inputs(case)
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa.fa_fwd_tiled(q, k, v, o, lse, scale=case["scale"], causal=case["causal"],
                    seqlens_k=sl, block_mask=bm, mask_block=case["mask_block"],
                    block_q=block_q)
    return o, lse


def _check(case, block_q, tag):
    _say(f"[tiled] block_q={block_q} {tag}")
    o, lse = _run(case, block_q)
    O, L = ref.forward(case["q"], case["k"], case["v"], **oracle_args(case))
    eo, el = maxabs(to_np(o), O), maxabs(to_np(lse), L)
    assert np.array_equal(np.isinf(to_np(lse)), np.isinf(L)), "dead rows differ"
    assert eo <= TOL["bf16"]["O"] and el <= TOL["bf16"]["L"], (eo, el)
    _say(f"[tiled] block_q={block_q} {tag} ok O={eo:.2e} L={el:.2e}")


@pytest.mark.parametrize("block_q", [64, 256])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 255, 256, 257, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_dense(block_q, N, causal):
    case = wl.random_case(2, 3, N, 64, seed=N + 3 * causal, causal=causal)
    _check(case, block_q, f"N={N} causal={causal}")


@pytest.mark.parametrize("block_q", [64, 256])
@pytest.mark.parametrize("masks", ["seqlens", "block", "both"])
def test_tiled_masks(block_q, masks):
    seqlens = "random" if masks in ("seqlens", "both") else None
    keep = 0.5 if masks in ("block", "both") else None
    case = wl.random_case(3, 2, 1100, 64, seed=31, causal=True, seqlens=seqlens,
                          block_keep_p=keep, mask_block=256)
    _check(case, block_q, f"masks={masks} mask_block=256")


def test_tiled_full_size_gpt2():
    w = wl.WORKLOADS["gpt2s_causal_b8h12n1024"]
    case = wl.make_inputs(w)
    case["mask_block"] = 128
    for bq in (64, 256):
        _check(case, bq, w.name)


def test_tile_128_is_fa_fwd():
    import torch
    import exact_io_aware_64_amd as fa
    case = wl.random_case(2, 2, 700, 64, seed=12, causal=True, seqlens="random")
    o, lse = _run(case, 128)
    q, k, v, _, sl, bm = device_inputs(case)
    o2, l2 = fa.forward(q, k, v, scale=case["scale"], causal=True, seqlens_k=sl)
    assert torch.equal(o, o2) and torch.equal(lse, l2)
