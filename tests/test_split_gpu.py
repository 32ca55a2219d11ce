"""GPU parity of the forward pass when each query tile's key range is split
over several groups of waves (fa_fwd_key_groups > 1: the grid has no more
query tiles than the GPU has CUs and the keys span >= 1024 rows), against the
fp64 oracle, for every mask kind, dropout, head dimensions 32/64/128,
separate query and key lengths, rows without visible keys, and tile lists
shorter than the number of groups."""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import attention_ref as ref
from oracle import dropout_ref as dref
from tests.gpu_util import TOL, excess_over, maxabs, opt_dev, relfro, to_dev, to_np

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(B, H, Nq, Nk, d=64, seed=0, seqlens=False, block_p=None):
    rng = np.random.default_rng(seed)
    q, do = wl.draw_tensors(rng, B, H, Nq, d, "bf16", count=2)
    k, v = wl.draw_tensors(rng, B, H, Nk, d, "bf16", count=2)
    sl = rng.integers(0, Nk + 1, size=B).astype(np.int32) if seqlens else None
    bm = None
    if block_p is not None:
        bm = (rng.random((-(-Nq // 128), -(-Nk // 128))) < block_p).astype(np.uint8)
    return dict(q=q, k=k, v=v, do=do, seqlens=sl, block_mask=bm, d=d)


def _groups(c):
    import exact_io_aware_64_amd as fa
    B, H, Nq, d = c["q"].shape
    return fa.fa_fwd_key_groups(fa.FA_BF16, B, H, Nq, c["k"].shape[2], d, 128)


def _check(c, causal, tag, p=0.0, backward=True):
    import torch
    import exact_io_aware_64_amd as fa
    groups = _groups(c)
    _say(f"[split] {tag} groups={groups}")
    assert groups == (2 if c["d"] == 128 else 3), "the shape must take the split path"
    tol = TOL["bf16"]
    scale = c["d"] ** -0.5
    q, k, v, do = (to_dev(c[n], "bf16") for n in ("q", "k", "v", "do"))
    sl, bm = opt_dev(c["seqlens"]), opt_dev(c["block_mask"])
    kw = dict(scale=scale, causal=causal, seqlens_k=sl, block_mask=bm, mask_block=128,
              dropout_p=p, seed=99, offset=1)
    o, lse = fa.forward(q, k, v, **kw)
    o2, lse2 = fa.forward(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "not repeatable"
    okw = dict(causal=causal, seqlens=c["seqlens"], block_mask=c["block_mask"], mask_block=128)
    if p > 0:
        O, L = dref.forward(c["q"], c["k"], c["v"], scale, p, 99, 1, **okw)
    else:
        O, L = ref.forward(c["q"], c["k"], c["v"], scale, **okw)
    errs = dict(O=maxabs(to_np(o), O), L=maxabs(to_np(lse), L))
    assert np.array_equal(np.isinf(to_np(lse)), np.isinf(L)), "dead rows differ"
    otol = tol["O"] * (256.0 / dref.keep_threshold(p) if p > 0 else 1.0)
    assert excess_over(to_np(o), O, otol) <= 0 and errs["L"] <= tol["L"], errs
    if backward:
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, **kw)
        if p > 0:
            g = dref.backward(c["q"], c["k"], c["v"], c["do"], scale, p, 99, 1, **okw)
        else:
            g = ref.backward(c["q"], c["k"], c["v"], c["do"], scale, **okw)
        for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), g):
            errs[name] = relfro(to_np(a), b)
            assert errs[name] <= tol["G"], (name, errs)
    _say(f"[split] {tag} ok {errs}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1024, 1500])
def test_split_dense(N, causal):
    _check(_case(1, 2, N, N, seed=N), causal, f"dense N={N} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_split_key_lengths(causal):
    _check(_case(3, 2, 1200, 1200, seed=5, seqlens=True), causal, f"seqlens causal={causal}")


@pytest.mark.parametrize("block_p", [0.08, 0.5])
@pytest.mark.parametrize("causal", [False, True])
def test_split_block_mask(block_p, causal):
    # at p = 0.08 most query tiles keep fewer 64-key tiles than there are
    # groups, and some keep none (rows without visible keys)
    _check(_case(1, 2, 2048, 2048, seed=7, block_p=block_p), causal,
           f"block mask p={block_p} causal={causal}")


def test_split_dropout():
    _check(_case(1, 2, 1100, 1100, seed=9), True, "dropout p=0.2", p=0.2)


@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_split_head_dims(d, causal):
    _check(_case(1, 2, 1300, 1300, d=d, seed=d), causal, f"d={d} causal={causal}")


@pytest.mark.parametrize("Nq,Nk", [(300, 3000), (1200, 1024), (1, 4096)])
def test_split_separate_lengths(Nq, Nk):
    # (1200, 1024) causal: the first 176 queries see no key
    _check(_case(2, 2, Nq, Nk, seed=Nq + Nk), True, f"Nq={Nq} Nk={Nk}")


def test_split_matches_unsplit_grid():
    """The same two heads inside a grid too large to split (288 query tiles):
    both runs meet the oracle, and differ by no more than rounding."""
    import torch
    import exact_io_aware_64_amd as fa
    c = _case(1, 24, 1500, 1500, seed=31)
    assert fa.fa_fwd_key_groups(fa.FA_BF16, 1, 24, 1500, 1500, 64, 128) == 1
    q, k, v = (to_dev(c[n], "bf16") for n in ("q", "k", "v"))
    o_big, l_big = fa.forward(q, k, v, scale=0.125, causal=True)
    o_two, l_two = fa.forward(q[:, :2].contiguous(), k[:, :2].contiguous(),
                              v[:, :2].contiguous(), scale=0.125, causal=True)
    torch.cuda.synchronize()
    O, L = ref.forward(c["q"][:, :2], c["k"][:, :2], c["v"][:, :2], 0.125, causal=True)
    for o, lse in ((o_big[:, :2], l_big[:, :2]), (o_two, l_two)):
        assert maxabs(to_np(o), O) <= TOL["bf16"]["O"]
        assert maxabs(to_np(lse), L) <= TOL["bf16"]["L"]
    assert maxabs(to_np(l_big[:, :2]), to_np(l_two)) <= 1e-5


def test_split_strided_layout_and_edge_lengths():
    """[B, N, H, d] storage (strided heads) and key lengths 0, 1 and N_k."""
    import exact_io_aware_64_amd as fa
    c = _case(3, 2, 1100, 1100, seed=41)
    c["seqlens"] = np.array([0, 1, 1100], np.int32)
    assert _groups(c) == 3
    tol = TOL["bf16"]
    q, k, v, do = (to_dev(c[n], "bf16", layout="bshd") for n in ("q", "k", "v", "do"))
    assert not q.is_contiguous()
    sl = opt_dev(c["seqlens"])
    kw = dict(scale=0.125, causal=False, seqlens_k=sl)
    o, lse = fa.forward(q, k, v, **kw)
    O, L = ref.forward(c["q"], c["k"], c["v"], 0.125, seqlens=c["seqlens"])
    assert np.array_equal(np.isinf(to_np(lse)), np.isinf(L)), "dead rows differ"
    assert excess_over(to_np(o), O, tol["O"]) <= 0
    assert maxabs(to_np(lse), L) <= tol["L"]
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, **kw)
    g = ref.backward(c["q"], c["k"], c["v"], c["do"], 0.125, seqlens=c["seqlens"])
    for a, b in zip((dq, dk, dv), g):
        assert relfro(to_np(a), b) <= tol["G"]
