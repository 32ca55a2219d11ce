"""GPU parity of fa_fwd_qk / fa_bwd_qk: N_q queries against N_k keys with the
causal mask aligned to the last query (key j visible to query i iff
j <= i + N_k - N_q), against the fp64 oracle."""
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


def _case(B, H, Nq, Nk, dtype="bf16", seed=0, seqlens=None, block_p=None, mask_block=128, d=64):
    rng = np.random.default_rng(seed)
    q, do = wl.draw_tensors(rng, B, H, Nq, d, dtype, count=2)
    k, v = wl.draw_tensors(rng, B, H, Nk, d, dtype, count=2)
    sl = None
    if seqlens == "random":
        sl = rng.integers(0, Nk + 1, size=B).astype(np.int32)
    bm = None
    if block_p is not None:
        tq, tk = -(-Nq // mask_block), -(-Nk // mask_block)
        bm = (rng.random((tq, tk)) < block_p).astype(np.uint8)
    return dict(q=q, k=k, v=v, do=do, seqlens=sl, block_mask=bm, mask_block=mask_block,
                dtype=dtype)


def _check(c, causal, tag, p=0.0, seed=5, offset=0, backward=True):
    import exact_io_aware_64_amd as fa
    _say(f"[qk] {tag}")
    dt = c["dtype"]
    tol = TOL[dt]
    q, k, v, do = (to_dev(c[n], dt) for n in ("q", "k", "v", "do"))
    sl, bm = opt_dev(c["seqlens"]), opt_dev(c["block_mask"])
    kw = dict(scale=0.125, causal=causal, seqlens_k=sl, block_mask=bm,
              mask_block=c["mask_block"], dropout_p=p, seed=seed, offset=offset)
    o, lse = fa.forward(q, k, v, **kw)
    okw = dict(causal=causal, seqlens=c["seqlens"], block_mask=c["block_mask"],
               mask_block=c["mask_block"])
    if p > 0:
        O, L = dref.forward(c["q"], c["k"], c["v"], 0.125, p, seed, offset, **okw)
    else:
        O, L = ref.forward(c["q"], c["k"], c["v"], 0.125, **okw)
    errs = dict(O=maxabs(to_np(o), O), L=maxabs(to_np(lse), L))
    assert np.array_equal(np.isinf(to_np(lse)), np.isinf(L)), "dead rows differ"
    # absolute budget (times the keep scale) plus the bf16 rounding of the stored
    # value itself: rows with few visible keys reach |O| > 4, whose half-ulp is 0.0156
    otol = tol["O"] * (256.0 / dref.keep_threshold(p) if p > 0 else 1.0)
    rel = 2.0 ** -8 if dt == "bf16" else 2.0 ** -24
    assert excess_over(to_np(o), O, otol, rel) <= 0 and errs["L"] <= tol["L"], errs
    if backward:
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, **kw)
        if p > 0:
            g = dref.backward(c["q"], c["k"], c["v"], c["do"], 0.125, p, seed, offset, **okw)
        else:
            g = ref.backward(c["q"], c["k"], c["v"], c["do"], 0.125, **okw)
        for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), g):
            errs[name] = relfro(to_np(a), b)
            assert np.all(np.isfinite(to_np(a)))
        for name in ("dQ", "dK", "dV"):
            assert errs[name] <= tol["G"], (name, errs)
    _say(f"[qk] {tag} ok {errs}")


SHAPES = [(1, 1000), (1, 64), (17, 129), (129, 17), (64, 1000), (300, 1024), (1000, 300),
          (128, 4096), (700, 700)]


@pytest.mark.parametrize("Nq,Nk", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_qk_dense(Nq, Nk, causal):
    _check(_case(2, 3, Nq, Nk, seed=Nq + 7 * Nk), causal, f"Nq={Nq} Nk={Nk} causal={causal}")


@pytest.mark.parametrize("Nq,Nk", [(33, 700), (700, 33), (256, 1100)])
@pytest.mark.parametrize("masks", ["seqlens", "block", "both"])
def test_qk_masks(Nq, Nk, masks):
    c = _case(3, 2, Nq, Nk, seed=Nq * Nk % 997, seqlens="random" if masks != "block" else None,
              block_p=0.5 if masks != "seqlens" else None)
    _check(c, True, f"Nq={Nq} Nk={Nk} masks={masks}")


@pytest.mark.parametrize("Nq,Nk", [(1, 300), (65, 300), (300, 65)])
@pytest.mark.parametrize("causal", [False, True])
def test_qk_f32(Nq, Nk, causal):
    _check(_case(2, 2, Nq, Nk, dtype="f32", seed=3), causal, f"f32 Nq={Nq} Nk={Nk}")


@pytest.mark.parametrize("Nq,Nk", [(100, 900), (900, 100)])
def test_qk_dropout(Nq, Nk):
    _check(_case(2, 2, Nq, Nk, seed=11), True, f"dropout Nq={Nq} Nk={Nk}", p=0.2, seed=77,
           offset=2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("Nq,Nk", [(100, 900), (900, 100)])
def test_qk_dropout_key_lengths_head_dims(dtype, d, Nq, Nk):
    c = _case(2, 2, Nq, Nk, dtype=dtype, seed=13 + d, seqlens="random", d=d)
    _check(c, True, f"dropout {dtype} d={d} Nq={Nq} Nk={Nk} key lengths", p=0.2, seed=78,
           offset=3)


def test_qk_decode_long_cache():
    """One query per head against 16K cached keys (B=2, H=8): forward only."""
    _check(_case(2, 8, 1, 16384, seed=21), True, "decode Nk=16384", backward=False)


def test_qk_square_is_the_plain_call():
    import torch
    import exact_io_aware_64_amd as fa
    c = _case(2, 2, 500, 500, seed=4)
    q, k, v = (to_dev(c[n], "bf16") for n in ("q", "k", "v"))
    o, lse = fa.forward(q, k, v, scale=0.125, causal=True)
    o2, l2 = torch.empty_like(o), torch.empty_like(lse)
    fa.fa_fwd_qk(q, k, v, o2, l2, scale=0.125, causal=True)
    assert torch.equal(o, o2) and torch.equal(lse, l2)
