"""GPU parity of attention with head dimensions 32 and 128, bf16 and fp32
(both kernel families are templated on d; d = 64 has its own tests), against
the fp64 oracle: edge lengths, causal, key lengths, tile masks, both layouts
and separate query / key lengths, for the forward and the backward pass
(dropout at these head dimensions is covered with the other dropout tests)."""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import attention_ref as ref
from tests.gpu_util import (TOL, device_inputs, gpu_forward, maxabs, oracle_args, opt_dev,
                            to_dev, to_np)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(case, tag, layout="bhsd"):
    _say(f"[headdim] {tag}")
    q, k, v, _, sl, bm = device_inputs(case, layout)
    o, lse = gpu_forward(case, q, k, v, sl, bm)
    O, L = ref.forward(case["q"], case["k"], case["v"], **oracle_args(case))
    eo, el = maxabs(to_np(o), O), maxabs(to_np(lse), L)
    tol = TOL[case["dtype"]]
    assert np.array_equal(np.isinf(to_np(lse)), np.isinf(L)), "dead rows differ"
    assert eo <= tol["O"] and el <= tol["L"], (eo, el)
    _say(f"[headdim] {tag} ok O={eo:.2e} L={el:.2e}")


DTYPES = ["bf16", "f32"]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("N", [1, 17, 63, 64, 65, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_headdim_dense(dtype, d, N, causal):
    case = wl.random_case(2, 3, N, d, dtype=dtype, seed=N + d + causal, causal=causal)
    _check(case, f"{dtype} d={d} N={N} causal={causal}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("masks", ["seqlens", "block", "both"])
def test_headdim_masks(dtype, d, masks):
    seqlens = "random" if masks in ("seqlens", "both") else None
    keep = 0.5 if masks in ("block", "both") else None
    case = wl.random_case(3, 2, 700, d, dtype=dtype, seed=d, causal=True, seqlens=seqlens,
                          block_keep_p=keep)
    _check(case, f"{dtype} d={d} masks={masks}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [32, 128])
def test_headdim_strided_layout(dtype, d):
    case = wl.random_case(2, 4, 257, d, dtype=dtype, seed=3 * d, causal=True)
    _check(case, f"{dtype} d={d} bshd", layout="bshd")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("Nq,Nk", [(1, 900), (200, 900), (900, 200)])
def test_headdim_separate_lengths(dtype, d, Nq, Nk):
    import exact_io_aware_64_amd as fa
    rng = np.random.default_rng(Nq + Nk + d)
    (q,) = wl.draw_tensors(rng, 2, 2, Nq, d, dtype, count=1)
    k, v = wl.draw_tensors(rng, 2, 2, Nk, d, dtype, count=2)
    _say(f"[headdim] {dtype} d={d} Nq={Nq} Nk={Nk}")
    o, lse = fa.forward(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype),
                        scale=d ** -0.5, causal=True)
    O, L = ref.forward(q, k, v, d ** -0.5, causal=True)
    eo, el = maxabs(to_np(o), O), maxabs(to_np(lse), L)
    assert eo <= TOL[dtype]["O"] and el <= TOL[dtype]["L"], (eo, el)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [32, 128])
def test_headdim_full_size(dtype, d):
    """B=4, H=16, N=2048 causal (a 7B-model-like attention shape for d=128)."""
    case = wl.random_case(4, 16, 2048, d, dtype=dtype, seed=99 + d, causal=True)
    rows = wl.sample_rows(np.random.default_rng(d), 4, 16, 2048, 256)
    _say(f"[headdim] full size {dtype} d={d}")
    q, k, v, _, sl, bm = device_inputs(case)
    o, lse = gpu_forward(case, q, k, v, sl, bm)
    O, L = ref.forward(case["q"], case["k"], case["v"], rows=rows, **oracle_args(case))
    idx = (np.arange(4)[:, None, None], np.arange(16)[None, :, None], rows)
    eo, el = maxabs(to_np(o)[idx], O), maxabs(to_np(lse)[idx], L)
    assert eo <= TOL[dtype]["O"] and el <= TOL[dtype]["L"], (eo, el)


def _check_bwd(case, tag):
    from tests.gpu_util import gpu_backward, relfro
    _say(f"[headdim bwd] {tag}")
    q, k, v, do, sl, bm = device_inputs(case)
    o, lse = gpu_forward(case, q, k, v, sl, bm)
    dq, dk, dv = gpu_backward(case, q, k, v, o, do, lse, sl, bm)
    g = ref.backward(case["q"], case["k"], case["v"], case["do"], **oracle_args(case))
    errs = {n: relfro(to_np(a), b) for n, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), g)}
    for n, e in errs.items():
        assert e <= TOL[case["dtype"]]["G"], (n, errs)
        assert np.all(np.isfinite(to_np(dict(dQ=dq, dK=dk, dV=dv)[n])))
    _say(f"[headdim bwd] {tag} ok {errs}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_headdim_backward_dense(dtype, d, N, causal):
    _check_bwd(wl.random_case(2, 2, N, d, dtype=dtype, seed=N + d + 5 * causal, causal=causal),
               f"{dtype} d={d} N={N} causal={causal}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("masks", ["seqlens", "block", "both"])
def test_headdim_backward_masks(dtype, d, masks):
    seqlens = "random" if masks in ("seqlens", "both") else None
    keep = 0.5 if masks in ("block", "both") else None
    _check_bwd(wl.random_case(3, 2, 700, d, dtype=dtype, seed=d + 1, causal=True,
                              seqlens=seqlens, block_keep_p=keep),
               f"{dtype} d={d} masks={masks}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [32, 128])
def test_headdim_backward_strided_layout(dtype, d):
    from tests.gpu_util import gpu_backward, relfro
    case = wl.random_case(2, 3, 257, d, dtype=dtype, seed=7 * d, causal=True)
    _say(f"[headdim bwd] {dtype} d={d} bshd")
    q, k, v, do, sl, bm = device_inputs(case, layout="bshd")
    o, lse = gpu_forward(case, q, k, v, sl, bm)
    grads = gpu_backward(case, q, k, v, o, do, lse, sl, bm)
    g = ref.backward(case["q"], case["k"], case["v"], case["do"], **oracle_args(case))
    for name, a, b in zip(("dQ", "dK", "dV"), grads, g):
        assert relfro(to_np(a), b) <= TOL[dtype]["G"], name


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("Nq,Nk", [(200, 900), (900, 200)])
def test_headdim_backward_separate_lengths(dtype, d, Nq, Nk):
    from tests.gpu_util import relfro
    import exact_io_aware_64_amd as fa
    rng = np.random.default_rng(Nq * 3 + Nk + d)
    q, do = wl.draw_tensors(rng, 2, 2, Nq, d, dtype, count=2)
    k, v = wl.draw_tensors(rng, 2, 2, Nk, d, dtype, count=2)
    _say(f"[headdim bwd] {dtype} d={d} Nq={Nq} Nk={Nk}")
    tq, tk, tv, tdo = (to_dev(x, dtype) for x in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, scale=d ** -0.5, causal=True)
    grads = fa.backward(tq, tk, tv, o, tdo, lse, scale=d ** -0.5, causal=True)
    g = ref.backward(q, k, v, do, d ** -0.5, causal=True)
    for name, a, b in zip(("dQ", "dK", "dV"), grads, g):
        assert relfro(to_np(a), b) <= TOL[dtype]["G"], name


def test_d128_workload_sampled():
    """The benchmarked d = 128 workload at full size, sampled rows."""
    w = wl.WORKLOADS["causal_b2h32n4096d128"]
    case = wl.make_inputs(w)
    case["mask_block"] = 128
    rows = case["rows"]
    _say(f"[headdim] {w.name} sampled")
    q, k, v, _, sl, bm = device_inputs(case)
    o, lse = gpu_forward(case, q, k, v, sl, bm)
    O, L = ref.forward(case["q"], case["k"], case["v"], rows=rows, **oracle_args(case))
    idx = (np.arange(w.B)[:, None, None], np.arange(w.H)[None, :, None], rows)
    eo, el = maxabs(to_np(o)[idx], O), maxabs(to_np(lse)[idx], L)
    assert eo <= TOL["bf16"]["O"] and el <= TOL["bf16"]["L"], (eo, el)
    _say(f"[headdim] {w.name} ok O={eo:.2e} L={el:.2e}")
