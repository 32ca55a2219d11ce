"""GPU parity: the HIP path (through the C ABI binding) against the fp64
oracle on the same seeded inputs.

Tolerances: O max-abs <= 1e-2, L max-abs <= 1e-3 and gradient relative
Frobenius error <= 1e-2 for bf16; 1e-5 for all of them in fp32.
"""
import functools
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import attention_ref as ref
from tests.gpu_util import (TOL, device_inputs, excess_over, gpu_backward, gpu_forward, maxabs,
                            opt_dev, oracle_args, relfro, to_dev, to_np)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_full(case, layout="bhsd", backward=True, tag="", o_rel=0.0):
    """Whole-tensor comparison with the oracle (small and medium sizes).
    o_rel > 0 adds o_rel |O*| to the O bound per element (the rounding of the
    stored value: 2^-8 for bf16 rows whose softmax sits on a few keys)."""
    _say(f"[parity] {tag} layout={layout}")
    tol = TOL[case["dtype"]]
    q, k, v, do, sl, bm = device_inputs(case, layout)
    o, lse = gpu_forward(case, q, k, v, sl, bm)
    O, L = ref.forward(case["q"], case["k"], case["v"], **oracle_args(case))
    eo = maxabs(to_np(o), O)
    el = maxabs(to_np(lse), L)
    assert np.array_equal(np.isinf(to_np(lse)), np.isinf(L)), "dead rows differ"
    if o_rel > 0:
        assert excess_over(to_np(o), O, tol["O"], o_rel) <= 0, f"O max-abs {eo}"
    else:
        assert eo <= tol["O"], f"O max-abs {eo}"
    assert el <= tol["L"], f"L max-abs {el}"
    errs = dict(O=eo, L=el)
    if backward:
        dq, dk, dv = gpu_backward(case, q, k, v, o, do, lse, sl, bm)
        gq, gk, gv = ref.backward(case["q"], case["k"], case["v"], case["do"],
                                  **oracle_args(case))
        for name, g, gs in (("dQ", dq, gq), ("dK", dk, gk), ("dV", dv, gv)):
            e = relfro(to_np(g), gs)
            errs[name] = e
            assert e <= tol["G"], f"{name} rel-Frobenius {e}"
            assert np.all(np.isfinite(to_np(g)))
    _say(f"[parity] {tag} ok {errs}")
    return errs


# ----------------------------------------------------------- the workloads

def test_single_head_f32_n128():
    w = wl.WORKLOADS["single_head_f32_n128"]
    case = wl.make_inputs(w)
    case["mask_block"] = 128
    check_full(case, tag=w.name, backward=True)


@pytest.mark.parametrize("name", ["gpt2s_causal_b8h12n1024", "bertl_padded_b16h16n512"])
def test_full_size_workload(name):
    w = wl.WORKLOADS[name]
    case = wl.make_inputs(w)
    case["mask_block"] = 128
    check_full(case, tag=name)


@functools.lru_cache(maxsize=1)
def _sampled_inputs(name):
    w = wl.WORKLOADS[name]
    case = wl.make_inputs(w)
    case["mask_block"] = 128
    return case


@pytest.mark.parametrize("name", ["long_causal_b1h16n16384", "blocksparse_b1h8n65536",
                                  "prefill_causal_b1h16q2048k16384",
                                  "train_causal_b2h16n4096d128",
                                  "train_causal_f32_b2h16n4096d128"])
def test_sampled_workload(name):
    """Full-size run checked on sampled query rows (O, L, dQ exact per row),
    a second backward with dO zeroed outside the sample (dK, dV exact for that
    restricted problem), and full-tensor gradient identities."""
    import torch
    _say(f"[parity] {name} sampled")
    case = _sampled_inputs(name)
    tol = TOL[case["dtype"]]
    rows = case["rows"]
    B, H, N, d = case["q"].shape
    q, k, v, do, sl, bm = device_inputs(case)
    o, lse = gpu_forward(case, q, k, v, sl, bm)
    dq, dk, dv = gpu_backward(case, q, k, v, o, do, lse, sl, bm)
    torch.cuda.synchronize()
    O, L = ref.forward(case["q"], case["k"], case["v"], rows=rows, **oracle_args(case))
    gq, gk, gv = ref.backward(case["q"], case["k"], case["v"], case["do"], rows=rows,
                              **oracle_args(case))
    o_np, l_np, dq_np = to_np(o), to_np(lse), to_np(dq)
    idx = (np.arange(B)[:, None, None], np.arange(H)[None, :, None], rows)
    eo = maxabs(o_np[idx], O)
    el = maxabs(l_np[idx], L)
    eq = relfro(dq_np[idx], gq)
    assert eo <= tol["O"], f"O {eo}"
    assert el <= tol["L"], f"L {el}"
    assert eq <= tol["G"], f"dQ {eq}"
    # full-tensor identities on the real run: sum_j dK_j = 0 and
    # sum_j dV_j = sum_i dO_i for every (b, h) (no row is fully masked here)
    dk_np, dv_np = to_np(dk), to_np(dv)
    do_sum = case["do"].astype(np.float64).sum(axis=2)
    for b in range(B):
        for h in range(H):
            assert np.linalg.norm(dk_np[b, h].sum(0)) <= 1e-2 * np.linalg.norm(dk_np[b, h])
            assert np.linalg.norm(dv_np[b, h].sum(0) - do_sum[b, h]) <= \
                1e-2 * np.linalg.norm(do_sum[b, h]) + 1e-2 * np.sqrt(N)
    # restricted problem: dO zero outside the sampled rows
    do_r = np.zeros_like(case["do"])
    for b in range(B):
        for h in range(H):
            do_r[b, h, rows[b, h]] = case["do"][b, h, rows[b, h]]
    dor = to_dev(do_r, case["dtype"])
    _, dk_r, dv_r = gpu_backward(case, q, k, v, o, dor, lse, sl, bm)
    ek = relfro(to_np(dk_r), gk)
    ev = relfro(to_np(dv_r), gv)
    assert ek <= tol["G"], f"dK {ek}"
    assert ev <= tol["G"], f"dV {ev}"
    _say(f"[parity] {name} ok O={eo:.3g} L={el:.3g} dQ={eq:.3g} dK={ek:.3g} dV={ev:.3g}")


# ------------------------------------------------------------ edge shapes

EDGE_N = [1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 300, 1000]


@pytest.mark.parametrize("N", EDGE_N)
@pytest.mark.parametrize("causal", [False, True])
def test_edge_lengths_dense(N, causal):
    case = wl.random_case(2, 2, N, 64, seed=N * 7 + causal, causal=causal)
    check_full(case, tag=f"N={N} causal={causal}")


@pytest.mark.parametrize("N", [17, 129, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masks", ["seqlens", "block", "both"])
def test_edge_masks(N, causal, masks):
    seqlens = "random" if masks in ("seqlens", "both") else None
    keep = 0.5 if masks in ("block", "both") else None
    case = wl.random_case(3, 2, N, 64, seed=N + 13 * causal, causal=causal, seqlens=seqlens,
                          block_keep_p=keep)
    check_full(case, tag=f"N={N} causal={causal} {masks}")


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_layouts(layout, dtype):
    case = wl.random_case(2, 3, 200, 64, dtype=dtype, seed=5, causal=True,
                          seqlens=[150, 200])
    check_full(case, layout=layout, tag=f"{dtype} {layout}")


@pytest.mark.parametrize("causal", [False, True])
def test_f32_masks(causal):
    case = wl.random_case(2, 2, 300, 64, dtype="f32", seed=3, causal=causal, seqlens="random",
                          block_keep_p=0.5)
    check_full(case, tag=f"f32 masks causal={causal}")


@pytest.mark.parametrize("N", [1, 17, 64, 65, 127, 128, 129, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_edge_lengths(N, causal):
    """fp32 forward (128-row workgroups on the fp32 matrix cores) and backward
    at lengths around its tile sizes."""
    case = wl.random_case(2, 2, N, 64, dtype="f32", seed=N * 5 + causal, causal=causal)
    check_full(case, tag=f"f32 N={N} causal={causal}")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mask_block", [256, 384])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_larger_mask_blocks(mask_block, dtype, causal, d):
    """Tile masks over 256 and 384 rows (each mask entry covers several of
    the kernels' 64- and 128-row tiles), with key lengths, forward and
    backward."""
    case = wl.random_case(2, 2, 1000, d, dtype=dtype, seed=mask_block + 7 * causal + d,
                          causal=causal, seqlens="random", block_keep_p=0.6,
                          mask_block=mask_block)
    check_full(case, tag=f"{dtype} d={d} mask_block={mask_block} causal={causal}")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("scale", [0.03, 0.4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_other_scales(scale, dtype, d):
    """Softmax scales other than 1/sqrt(d): nearly flat (0.03) and sharp (0.4)
    distributions, causal with key lengths, forward and backward.  A sharp
    softmax puts rows on one or a few keys, |O| up to the largest |v| (> 4),
    where half an ulp of the stored bf16 value exceeds a flat 1e-2: O is
    held to 1e-2 + 2^-8 |O*| there, as for dropout and N_q != N_k."""
    case = wl.random_case(2, 2, 500, d, dtype=dtype, seed=int(scale * 100) + d, causal=True,
                          seqlens="random", scale=scale)
    check_full(case, tag=f"{dtype} d={d} scale={scale}",
               o_rel=2.0 ** -8 if dtype == "bf16" else 0.0)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_key_lengths_zero_and_full(dtype, d):
    """len 0 (every row fully masked: O = 0, L = -inf, zero gradients), len 1
    and len N in one batch."""
    case = wl.random_case(3, 2, 200, d, dtype=dtype, seed=9, seqlens=[0, 1, 200])
    check_full(case, tag=f"{dtype} d={d} seqlens 0/1/N")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_empty_block_mask_rows(dtype, d):
    rng = np.random.default_rng(4)
    case = wl.random_case(1, 2, 512, d, dtype=dtype, seed=4)
    bm = (rng.random((4, 4)) < 0.5).astype(np.uint8)
    bm[1, :] = 0      # query tile 1 sees nothing
    bm[:, 3] = 0      # key tile 3 is seen by nobody (zero dK, dV)
    case["block_mask"] = bm
    check_full(case, tag=f"{dtype} d={d} empty mask row/column")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_mask_all_ones_equals_dense(dtype, d):
    case = wl.random_case(1, 2, 384, d, dtype=dtype, seed=8, causal=True)
    q, k, v, do, _, _ = device_inputs(case)
    o1, l1 = gpu_forward(case, q, k, v, None, None)
    ones = opt_dev(np.ones((3, 3), np.uint8))
    o2, l2 = gpu_forward(case, q, k, v, None, ones)
    assert np.array_equal(to_np(o1), to_np(o2)) and np.array_equal(to_np(l1), to_np(l2))


def _product_magnitudes(q, k, v, do, scale):
    """Element-wise magnitudes |A||B| of the three gradient products, used to
    bound rounding error when the exact gradient itself vanishes."""
    q, k, v, do = (np.asarray(x, np.float64)[0, 0] for x in (q, k, v, do))
    s = scale * q @ k.T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return (scale * np.abs(ds) @ np.abs(k), scale * np.abs(ds).T @ np.abs(q),
            np.abs(p).T @ np.abs(do))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["plus", "minus", "mixed"])
def test_huge_scores_stay_finite(kind, dtype, d):
    """Scores of +-312.5 d for every pair (+-20000 at d = 64; the overflow /
    underflow examples of the safe-softmax discussion): results stay finite
    and match the oracle.  L is checked to a few fp32 ulps at its magnitude.
    With all keys equal the exact dQ is 0 while fp32 scores that large carry
    ~1e-3 absolute error, so gradients are bounded relative to the magnitude
    of their products, ||g - g*|| <= 1e-2 || |A| |B| ||."""
    N = 256
    q = np.full((1, 1, N, d), 50.0, np.float32)
    k = np.full((1, 1, N, d), 50.0 if kind != "minus" else -50.0, np.float32)
    if kind == "mixed":
        k[0, 0, 1::2] = -50.0
    rng = np.random.default_rng(0)
    v = wl.round_to_bf16(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    do = wl.round_to_bf16(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    case = dict(q=q, k=k, v=v, do=do, scale=0.125, causal=False, dtype=dtype,
                seqlens=None, block_mask=None)
    qd, kd, vd, dod, _, _ = device_inputs(case)
    o, lse = gpu_forward(case, qd, kd, vd, None, None)
    O, L = ref.forward(q, k, v, 0.125)
    assert np.all(np.isfinite(to_np(o))) and np.all(np.isfinite(to_np(lse)))
    assert maxabs(to_np(o), O) <= 1e-2
    assert maxabs(to_np(lse), L) <= 8 * np.spacing(np.float32(312.5 * d)) + 1e-3
    dq, dk, dv = gpu_backward(case, qd, kd, vd, o, dod, lse, None, None)
    gq, gk, gv = ref.backward(q, k, v, do, 0.125)
    mags = _product_magnitudes(q, k, v, do, 0.125)
    for name, g, gs, mag in zip(("dQ", "dK", "dV"), (dq, dk, dv), (gq, gk, gv), mags):
        gn = to_np(g)
        assert np.all(np.isfinite(gn)), name
        err = np.linalg.norm(gn[0, 0] - gs[0, 0])
        assert err <= 1e-2 * np.linalg.norm(mag), (name, err, np.linalg.norm(mag))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_repeatable_bitwise(dtype, d):
    """No atomics anywhere: two runs give identical bits."""
    case = wl.random_case(2, 4, 700, d, dtype=dtype, seed=21, causal=True, seqlens="random")
    q, k, v, do, sl, bm = device_inputs(case)
    r1 = gpu_forward(case, q, k, v, sl, bm)
    r2 = gpu_forward(case, q, k, v, sl, bm)
    g1 = gpu_backward(case, q, k, v, r1[0], do, r1[1], sl, bm)
    g2 = gpu_backward(case, q, k, v, r1[0], do, r1[1], sl, bm)
    for a, b in zip(r1 + g1, r2 + g2):
        assert np.array_equal(to_np(a), to_np(b))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_halves_equal_full_call(dtype, d):
    """fa_bwd_dkdv and fa_bwd_dq are independent (dK/dV first here, with no
    dQ call before it) and together give exactly what fa_bwd gives."""
    import torch
    import exact_io_aware_64_amd as fa
    case = wl.random_case(2, 3, 333, d, dtype=dtype, seed=31, causal=True, seqlens="random",
                          block_keep_p=0.6)
    q, k, v, do, sl, bm = device_inputs(case)
    o, lse = gpu_forward(case, q, k, v, sl, bm)
    g1 = gpu_backward(case, q, k, v, o, do, lse, sl, bm)
    kw = dict(scale=case["scale"], causal=case["causal"], seqlens_k=sl, block_mask=bm,
              mask_block=128)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    fa.fa_bwd_dkdv(q, k, v, o, do, lse, dk, dv, **kw)
    fa.fa_bwd_dq(q, k, v, o, do, lse, dq, **kw)
    for a, b in zip(g1, (dq, dk, dv)):
        assert np.array_equal(to_np(a), to_np(b))


def test_prepared_calls_equal_direct_calls():
    """The binding's prepared calls (arguments converted once) launch exactly
    what the direct calls launch."""
    import torch
    import exact_io_aware_64_amd as fa
    case = wl.random_case(2, 2, 257, 64, seed=41, causal=True, seqlens="random")
    q, k, v, do, sl, bm = device_inputs(case)
    o1, l1 = gpu_forward(case, q, k, v, sl, bm)
    g1 = gpu_backward(case, q, k, v, o1, do, l1, sl, bm)
    kw = dict(scale=case["scale"], causal=True, seqlens_k=sl, block_mask=bm)
    o2, l2 = torch.empty_like(q), torch.empty_like(l1)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    fa.prepare_fwd(q, k, v, o2, l2, **kw)()
    fa.prepare_bwd(q, k, v, o2, do, l2, dq, dk, dv, **kw)()
    for a, b in zip((o1, l1) + tuple(g1), (o2, l2, dq, dk, dv)):
        assert np.array_equal(to_np(a), to_np(b))


def test_memory_linear_in_N():
    """Peak device memory of fwd + bwd is the inputs, outputs, L and the
    per-row workspace: linear in N, nothing N x N (at N = 65536 one bf16
    score matrix for 8 heads would be 68.7 GB)."""
    import torch
    import exact_io_aware_64_amd as fa
    H, d = 8, 64
    peaks = {}
    for N in (4096, 16384, 65536):
        case = wl.random_case(1, H, 256, d, seed=1)   # values irrelevant here
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        q = torch.randn(1, H, N, d, device="cuda", dtype=torch.bfloat16)
        k, v, do = torch.randn_like(q), torch.randn_like(q), torch.randn_like(q)
        bm = torch.eye(N // 128, dtype=torch.uint8, device="cuda")
        o, lse = fa.forward(q, k, v, scale=0.125, block_mask=bm)
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale=0.125, block_mask=bm)
        torch.cuda.synchronize()
        peaks[N] = torch.cuda.max_memory_allocated() - base
        expect = 8 * H * N * d * 2 + 2 * H * N * 4 + (N // 128) ** 2
        assert peaks[N] <= 1.1 * expect + (4 << 20), (N, peaks[N], expect)
        del q, k, v, do, o, lse, dq, dk, dv, bm, case
    _say(f"[memory] peaks {peaks}")


@pytest.mark.parametrize("B,H", [(5, 8), (3, 8), (2, 12), (3, 5)])
def test_noncausal_head_groups(B, H):
    """Non-causal backward grids take each XCD's heads (B*H / 8 of them when
    B*H is a multiple of 8) in groups of four: 5, 3 and 3 heads per XCD give
    a short last group or a single one; B*H = 15 takes the plain order."""
    case = wl.random_case(B, H, 300, 64, seed=B * 100 + H, causal=False, seqlens="random",
                          block_keep_p=0.7)
    check_full(case, tag=f"non-causal head groups B={B} H={H}")
