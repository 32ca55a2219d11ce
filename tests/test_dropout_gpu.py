"""GPU parity of attention with dropout (fa_fwd_dropout / fa_bwd_dropout)
against the fp64 dropout oracle.

The keep mask is checked bit for bit through every kernel path that
regenerates it, with inputs that make each pair's keep bit readable in an
output:
  * forward: Q = 0 makes P uniform over the visible keys, and V one-hot over
    a window of 64 keys gives O_i[c] = s Z_{i, j0+c} / n_i;
  * dK/dV role, P path: dO one-hot over a window of 64 queries gives
    dV_j[c] = s Z_{i0+c, j} P_{i0+c, j};
  * dQ role: with dO_i . v_j = 1, dS_ij = P_ij (s Z_ij - D_i) with
    0 < D_i < s, so K one-hot over a key window makes the sign of dQ_i[c]
    the keep bit of (i, j0+c);
  * dK/dV role, dS path: the same with K = 0 and Q one-hot over a query
    window, read from the sign of dK.
Random inputs are then compared with the oracle to the usual tolerances,
except for O: each element may differ by the plain bound times the keep
scale s = 256 / t (kept values are s times larger) plus the rounding of the
stored bf16 value itself, 2^-8 of its magnitude (a row with a single visible
key reaches |O| = s |v|, whose half-ulp exceeds the plain bound once it
passes 4).
"""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import dropout_ref as dref
from tests.gpu_util import (TOL, device_inputs, excess_over, maxabs, opt_dev, relfro, to_dev,
                            to_np)

pytestmark = pytest.mark.gpu

SEED = 0x9E3779B97F4A7C15  # both key words nonzero
OFFSET = 5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _fa():
    import exact_io_aware_64_amd as fa
    return fa


def _oracle_keep(B, H, N, p, seed=SEED, offset=OFFSET):
    """bool [B, H, N, N]: the oracle's keep bits."""
    z = np.zeros((B, H, N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            z[b, h] = dref.keep_mask(np.arange(N), N, b * H + h, p, seed, offset)
    return z


def _visible(B, N, causal, seqlens):
    vis = np.ones((B, N, N), dtype=bool)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    for b in range(B):
        if causal:
            vis[b] &= j <= i
        if seqlens is not None:
            vis[b] &= j < seqlens[b]
    return vis


def _zeros(B, H, N, d=64):
    return np.zeros((B, H, N, d), np.float32)


# (dtype, head dimension): every pair the library builds
DTYPE_D = [("bf16", 64), ("f32", 64), ("bf16", 32), ("bf16", 128), ("f32", 32), ("f32", 128)]


@pytest.mark.parametrize("dtype,d", DTYPE_D)
@pytest.mark.parametrize("causal,padded", [(False, False), (True, False), (True, True)])
def test_keep_mask_bit_exact_forward_and_dv(dtype, d, causal, padded):
    fa = _fa()
    import torch
    B, H, N, p = 2, 3, 300, 0.5
    seqlens = np.array([300, 211], np.int32) if padded else None
    sl = opt_dev(seqlens)
    vis = _visible(B, N, causal, seqlens)
    z = _oracle_keep(B, H, N, p)
    _say(f"[dropout mask fwd/dv] {dtype} d={d} causal={causal} padded={padded}")
    zero = _zeros(B, H, N, d)
    q0 = to_dev(zero, dtype)
    kw = dict(scale=0.125, causal=causal, seqlens_k=sl, dropout_p=p, seed=SEED, offset=OFFSET)
    got_f = np.zeros((B, H, N, N), dtype=bool)
    got_b = np.zeros((B, H, N, N), dtype=bool)
    win = min(64, d)  # keys (queries) read back per call: one per output column
    for w0 in range(0, N, win):
        wn = min(win, N - w0)
        onehot = np.zeros((B, H, N, d), np.float32)
        onehot[:, :, w0:w0 + wn, :][:, :, np.arange(wn), np.arange(wn)] = 1.0
        oh = to_dev(onehot, dtype)
        # forward: V one-hot over keys w0 .. w0 + wn
        o, lse = fa.forward(q0, q0, oh, **kw)
        got_f[:, :, :, w0:w0 + wn] = to_np(o)[:, :, :, :wn] > 0
        # backward, dV: dO one-hot over queries w0 .. w0 + wn
        o2, lse2 = fa.forward(q0, q0, q0, **kw)
        dq, dk, dv = fa.backward(q0, q0, q0, o2, oh, lse2, **kw)
        got_b[:, :, w0:w0 + wn, :] = np.transpose(to_np(dv)[:, :, :, :wn], (0, 1, 3, 2)) > 0
        torch.cuda.synchronize()
    want = z & vis[:, None]
    assert np.array_equal(got_f, want), f"forward: {np.sum(got_f != want)} pairs differ"
    assert np.array_equal(got_b, want), f"dV: {np.sum(got_b != want)} pairs differ"
    _say(f"[dropout mask fwd/dv] ok, kept {want.sum()} of {vis.sum() * H} visible pairs")


@pytest.mark.parametrize("dtype,d", DTYPE_D)
def test_keep_mask_bit_exact_dq_and_dk_signs(dtype, d):
    fa = _fa()
    import torch
    B, H, N, p = 2, 2, 300, 0.5
    z = _oracle_keep(B, H, N, p)
    _say(f"[dropout mask dq/dk] {dtype} d={d}")
    zero = _zeros(B, H, N, d)
    z0 = to_dev(zero, dtype)
    e0 = np.zeros((B, H, N, d), np.float32)
    e0[..., 0] = 1.0
    ones0 = to_dev(e0, dtype)  # v_j = dO_i = e_0, so dO_i . v_j = 1
    kw = dict(scale=0.125, causal=False, dropout_p=p, seed=SEED, offset=OFFSET)
    sign_q = np.zeros((B, H, N, N), dtype=np.int8)
    sign_k = np.zeros((B, H, N, N), dtype=np.int8)
    win = min(64, d)
    for w0 in range(0, N, win):
        wn = min(win, N - w0)
        onehot = np.zeros((B, H, N, d), np.float32)
        onehot[:, :, w0:w0 + wn, :][:, :, np.arange(wn), np.arange(wn)] = 1.0
        oh = to_dev(onehot, dtype)
        # dQ role: Q = 0, K one-hot over keys w0 ..
        o, lse = fa.forward(z0, oh, ones0, **kw)
        dq, _, _ = fa.backward(z0, oh, ones0, o, ones0, lse, **kw)
        sign_q[:, :, :, w0:w0 + wn] = np.sign(to_np(dq)[:, :, :, :wn])
        # dK/dV role: K = 0, Q one-hot over queries w0 ..
        o, lse = fa.forward(oh, z0, ones0, **kw)
        _, dk, _ = fa.backward(oh, z0, ones0, o, ones0, lse, **kw)
        sign_k[:, :, w0:w0 + wn, :] = np.transpose(np.sign(to_np(dk)[:, :, :, :wn]), (0, 1, 3, 2))
        torch.cuda.synchronize()
    # every row keeps some but not all of its 300 keys, so no sign is zero
    want = np.where(z, 1, -1).astype(np.int8)
    assert np.array_equal(sign_q, want), f"dQ: {np.sum(sign_q != want)} pairs differ"
    assert np.array_equal(sign_k, want), f"dK: {np.sum(sign_k != want)} pairs differ"
    _say("[dropout mask dq/dk] ok")


def _keep_scale(p):
    return 256.0 / dref.keep_threshold(p)


def _check_random(case, p, seed, offset, tag):
    fa = _fa()
    _say(f"[dropout parity] {tag}")
    tol = TOL[case["dtype"]]
    q, k, v, do, sl, bm = device_inputs(case)
    okw = dict(causal=case["causal"], seqlens=case["seqlens"], block_mask=case["block_mask"],
               mask_block=case["mask_block"])
    kw = dict(scale=case["scale"], causal=case["causal"], seqlens_k=sl, block_mask=bm,
              mask_block=case["mask_block"], dropout_p=p, seed=seed, offset=offset)
    o, lse = fa.forward(q, k, v, **kw)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, **kw)
    O, L = dref.forward(case["q"], case["k"], case["v"], case["scale"], p, seed, offset, **okw)
    gq, gk, gv = dref.backward(case["q"], case["k"], case["v"], case["do"], case["scale"], p,
                               seed, offset, **okw)
    errs = dict(O=maxabs(to_np(o), O), L=maxabs(to_np(lse), L))
    for name, g, gs in (("dQ", dq, gq), ("dK", dk, gk), ("dV", dv, gv)):
        errs[name] = relfro(to_np(g), gs)
    _say(f"[dropout parity] {tag} {errs}")
    # the rounding of the stored value: half an ulp of bf16 or of fp32
    rel = 2.0 ** -8 if case["dtype"] == "bf16" else 2.0 ** -24
    assert excess_over(to_np(o), O, tol["O"] * _keep_scale(p), rel) <= 0, errs
    assert errs["L"] <= tol["L"], errs
    for name in ("dQ", "dK", "dV"):
        assert errs[name] <= tol["G"], (name, errs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N", [17, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_parity_dense(dtype, N, causal):
    case = wl.random_case(2, 2, N, 64, dtype=dtype, seed=N + causal, causal=causal)
    _check_random(case, 0.1, SEED + N, 3, f"{dtype} N={N} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("N", [17, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_parity_head_dims(dtype, d, N, causal):
    case = wl.random_case(2, 2, N, d, dtype=dtype, seed=N + d + causal, causal=causal)
    _check_random(case, 0.1, SEED + N + d, 3, f"{dtype} d={d} N={N} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("masks", ["seqlens", "block", "both"])
def test_dropout_parity_head_dims_masks(dtype, d, masks):
    seqlens = "random" if masks in ("seqlens", "both") else None
    keep = 0.5 if masks in ("block", "both") else None
    case = wl.random_case(3, 2, 640, d, dtype=dtype, seed=31 + d, causal=True,
                          seqlens=seqlens, block_keep_p=keep)
    _check_random(case, 0.3, 777, 2, f"{dtype} d={d} masks={masks}")


@pytest.mark.parametrize("masks", ["seqlens", "block", "both"])
def test_dropout_parity_masks(masks):
    seqlens = "random" if masks in ("seqlens", "both") else None
    keep = 0.5 if masks in ("block", "both") else None
    case = wl.random_case(3, 2, 640, 64, seed=21, causal=True, seqlens=seqlens,
                          block_keep_p=keep)
    _check_random(case, 0.3, 12345, 0, f"masks={masks}")


def test_zero_probability_is_the_plain_call():
    fa = _fa()
    import torch
    case = wl.random_case(2, 2, 300, 64, seed=2, causal=True)
    q, k, v, do, _, _ = device_inputs(case)
    o0, l0 = fa.forward(q, k, v, scale=0.125, causal=True)
    o1, l1 = fa.forward(q, k, v, scale=0.125, causal=True, dropout_p=0.0, seed=7)
    o2 = torch.empty_like(o0)
    l2 = torch.empty_like(l0)
    fa.fa_fwd_dropout(q, k, v, o2, l2, scale=0.125, causal=True, dropout_p=0.0, seed=7)
    assert torch.equal(o0, o1) and torch.equal(o0, o2) and torch.equal(l0, l2)
    g0 = fa.backward(q, k, v, o0, do, l0, scale=0.125, causal=True)
    g2 = [torch.empty_like(q) for _ in range(3)]
    fa.fa_bwd_dropout(q, k, v, o0, do, l0, *g2, scale=0.125, causal=True, dropout_p=0.0,
                      seed=7)
    for a, b in zip(g0, g2):
        assert torch.equal(a, b)


def test_same_seed_repeats_and_offset_changes_the_mask():
    fa = _fa()
    import torch
    case = wl.random_case(1, 2, 256, 64, seed=6)
    q, k, v, do, _, _ = device_inputs(case)
    kw = dict(scale=0.125, dropout_p=0.2, seed=99)
    a, la = fa.forward(q, k, v, offset=0, **kw)
    b, lb = fa.forward(q, k, v, offset=0, **kw)
    c, lc = fa.forward(q, k, v, offset=1, **kw)
    assert torch.equal(a, b) and torch.equal(la, lb)
    assert not torch.equal(a, c)
    # L is the statistic of the undropped softmax
    plain_o, plain_l = fa.forward(q, k, v, scale=0.125)
    assert maxabs(to_np(la), to_np(plain_l)) <= 1e-6
    assert maxabs(to_np(lc), to_np(plain_l)) <= 1e-6


def test_sampled_full_size_gpt2_with_dropout():
    """GPT-2 small shape (B=8, H=12, N=1024, causal, bf16) with p = 0.1:
    O, L and dQ on 128 sampled rows per head; dK, dV of the problem whose dO
    is zero outside the sample."""
    fa = _fa()
    w = wl.WORKLOADS["gpt2s_causal_b8h12n1024"]
    case = wl.make_inputs(w)
    rng = np.random.default_rng(77)
    rows = wl.sample_rows(rng, w.B, w.H, w.N, 128)
    p, seed, offset = 0.1, 2024, 1
    _say("[dropout sampled] gpt2s_causal_b8h12n1024 p=0.1")
    q, k, v, do, _, _ = device_inputs(dict(case, dtype="bf16"))
    kw = dict(scale=w.scale, causal=True, dropout_p=p, seed=seed, offset=offset)
    o, lse = fa.forward(q, k, v, **kw)
    dq, _, _ = fa.backward(q, k, v, o, do, lse, **kw)
    O, L = dref.forward(case["q"], case["k"], case["v"], w.scale, p, seed, offset, causal=True,
                        rows=rows)
    do_r = np.zeros_like(case["do"])
    for b in range(w.B):
        for h in range(w.H):
            do_r[b, h, rows[b, h]] = case["do"][b, h, rows[b, h]]
    gq, gk, gv = dref.backward(case["q"], case["k"], case["v"], do_r, w.scale, p, seed, offset,
                               causal=True, rows=rows)
    idx = (np.arange(w.B)[:, None, None], np.arange(w.H)[None, :, None], rows)
    errs = dict(O=maxabs(to_np(o)[idx], O), L=maxabs(to_np(lse)[idx], L),
                dQ=relfro(to_np(dq)[idx], gq))
    _, dk_r, dv_r = fa.backward(q, k, v, o, to_dev(do_r, "bf16"), lse, **kw)
    errs["dK"] = relfro(to_np(dk_r), gk)
    errs["dV"] = relfro(to_np(dv_r), gv)
    _say(f"[dropout sampled] {errs}")
    tol = TOL["bf16"]
    assert excess_over(to_np(o)[idx], O, tol["O"] * _keep_scale(p)) <= 0, errs
    assert errs["L"] <= tol["L"], errs
    for name in ("dQ", "dK", "dV"):
        assert errs[name] <= tol["G"], (name, errs)


@pytest.mark.parametrize("name", ["train_causal_b2h16n4096d128",
                                  "train_causal_f32_b2h16n4096d128"])
def test_sampled_full_size_d128_training_with_dropout(name):
    """Causal training shape with head dimension 128 (B=2, H=16, N=4096, bf16
    and fp32) with p = 0.1: O, L and dQ on 128 sampled rows per head; dK, dV
    of the problem whose dO is zero outside the sample."""
    fa = _fa()
    w = wl.WORKLOADS[name]
    case = wl.make_inputs(w)
    rows = case["rows"][:, :, :128]
    p, seed, offset = 0.1, 2024, 0
    _say(f"[dropout sampled] {name} p=0.1")
    q, k, v, do, _, _ = device_inputs(case)
    kw = dict(scale=w.scale, causal=True, dropout_p=p, seed=seed, offset=offset)
    o, lse = fa.forward(q, k, v, **kw)
    dq, _, _ = fa.backward(q, k, v, o, do, lse, **kw)
    O, L = dref.forward(case["q"], case["k"], case["v"], w.scale, p, seed, offset, causal=True,
                        rows=rows)
    do_r = np.zeros_like(case["do"])
    for b in range(w.B):
        for h in range(w.H):
            do_r[b, h, rows[b, h]] = case["do"][b, h, rows[b, h]]
    gq, gk, gv = dref.backward(case["q"], case["k"], case["v"], do_r, w.scale, p, seed, offset,
                               causal=True, rows=rows)
    idx = (np.arange(w.B)[:, None, None], np.arange(w.H)[None, :, None], rows)
    errs = dict(O=maxabs(to_np(o)[idx], O), L=maxabs(to_np(lse)[idx], L),
                dQ=relfro(to_np(dq)[idx], gq))
    _, dk_r, dv_r = fa.backward(q, k, v, o, to_dev(do_r, w.dtype), lse, **kw)
    errs["dK"] = relfro(to_np(dk_r), gk)
    errs["dV"] = relfro(to_np(dv_r), gv)
    _say(f"[dropout sampled d128] {errs}")
    tol = TOL[w.dtype]
    rel = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -24
    assert excess_over(to_np(o)[idx], O, tol["O"] * _keep_scale(p), rel) <= 0, errs
    assert errs["L"] <= tol["L"], errs
    for name in ("dQ", "dK", "dV"):
        assert errs[name] <= tol["G"], (name, errs)
