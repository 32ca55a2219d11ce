"""fa_bwd_noalloc, the backward entry point that allocates nothing (its D
rows live in a scratch array inside the library), against fa_bwd and the
fp64 oracle: several calls in a row on one GPU, each smaller than the one
before, so later calls run over a scratch array that still holds an earlier
call's values."""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import attention_ref as ref
from tests.gpu_util import TOL, device_inputs, oracle_args, relfro, to_np

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# (B, H, N, d, causal, key lengths, tile-mask keep probability), largest first
CALLS = [
    (2, 4, 1000, 64, True, None, None),
    (3, 2, 300, 64, False, "random", 0.5),
    (1, 3, 200, 128, True, None, None),
    (2, 1, 130, 32, False, "random", None),
]


def test_noalloc_matches_fa_bwd_on_calls_in_a_row():
    import torch
    import exact_io_aware_64_amd as fa
    for i, (B, H, N, d, causal, seqlens, keep) in enumerate(CALLS):
        case = wl.random_case(B, H, N, d, seed=100 + i, causal=causal, seqlens=seqlens,
                              block_keep_p=keep)
        _say(f"[noalloc] call {i}: B={B} H={H} N={N} d={d} causal={causal} "
             f"seqlens={seqlens} keep={keep}")
        q, k, v, do, sl, bm = device_inputs(case)
        kw = dict(scale=case["scale"], causal=causal, seqlens_k=sl, block_mask=bm,
                  mask_block=case["mask_block"])
        o, lse = fa.forward(q, k, v, **kw)
        want = fa.backward(q, k, v, o, do, lse, **kw)
        got = [torch.full_like(t, float("nan")) for t in want]
        fa.fa_bwd_noalloc(q, k, v, o, do, lse, *got, **kw)
        torch.cuda.synchronize()
        # the same kernels on the same D: identical to fa_bwd bit for bit
        for name, g, w in zip(("dQ", "dK", "dV"), got, want):
            assert torch.equal(g, w), f"call {i}: {name} differs from fa_bwd"
        # and within the parity tolerance of the oracle
        G = ref.backward(case["q"], case["k"], case["v"], case["do"], **oracle_args(case))
        errs = {name: relfro(to_np(g), gs) for name, g, gs in zip(("dQ", "dK", "dV"), got, G)}
        _say(f"[noalloc] call {i} ok {errs}")
        for name, e in errs.items():
            assert e <= TOL["bf16"]["G"], (i, name, e)
            assert np.all(np.isfinite(to_np(got[("dQ", "dK", "dV").index(name)])))
