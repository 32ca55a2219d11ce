"""Pins for the fp64 oracle: every check here comes from something other than
the oracle's own formula -- a hand-worked example, closed forms, invariants of
softmax attention, central finite differences, the pages' online-softmax
procedure, and a float64 library cross-check."""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_ref as ref
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MASK_KINDS = ["none", "causal", "padded", "block", "causal_padded_block"]


def _case(kind, B=1, H=2, N=12, d=4, seed=0, mask_block=4):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    causal = kind in ("causal", "causal_padded_block")
    seqlens = None
    block = None
    if kind in ("padded", "causal_padded_block"):
        seqlens = rng.integers(max(1, N // 2), N + 1, size=B).astype(np.int32)
    if kind in ("block", "causal_padded_block"):
        block = wl.draw_block_mask(rng, N, 0.4, mask_block)
    return dict(q=q, k=k, v=v, do=do, scale=0.7, causal=causal, seqlens=seqlens,
                block_mask=block, mask_block=mask_block)


def _fwd(c, **over):
    a = dict(c)
    a.update(over)
    return ref.forward(a["q"], a["k"], a["v"], a["scale"], a["causal"], a["seqlens"],
                       a["block_mask"], a["mask_block"])


def _bwd(c, **over):
    a = dict(c)
    a.update(over)
    return ref.backward(a["q"], a["k"], a["v"], a["do"], a["scale"], a["causal"],
                        a["seqlens"], a["block_mask"], a["mask_block"])


# ---------------------------------------------------------------- hand-worked

@pytest.mark.parametrize("variant", ["noncausal", "causal"])
def test_hand_worked_fixture(variant):
    with open(os.path.join(GOLDEN, "hand_n2_d1.json")) as f:
        g = json.load(f)
    q = np.array([math.log(3.0), 0.0]).reshape(1, 1, 2, 1)
    k = np.array([0.0, 1.0]).reshape(1, 1, 2, 1)
    v = np.array([1.0, 5.0]).reshape(1, 1, 2, 1)
    do = np.ones((1, 1, 2, 1))
    causal = variant == "causal"
    O, L = ref.forward(q, k, v, 1.0, causal)
    dq, dk, dv = ref.backward(q, k, v, do, 1.0, causal)
    exp = g[variant]["values"]
    np.testing.assert_allclose(O.ravel(), exp["O"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(L.ravel(), exp["L"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv.ravel(), exp["dV"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dq.ravel(), exp["dQ"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk.ravel(), exp["dK"], rtol=0, atol=1e-14)


# ------------------------------------------------------------- forward pins

@pytest.mark.parametrize("kind", MASK_KINDS)
def test_identity_values_expose_P_rows(kind):
    """With V = I (d = N) the output rows are the rows of P: non-negative,
    zero on masked keys and summing to one on every row with a visible key."""
    c = _case(kind, N=16, d=16)
    B, H, N, _ = c["q"].shape
    v = np.broadcast_to(np.eye(N), (B, H, N, N)).copy()
    O, L = _fwd(c, v=v)
    for b in range(B):
        sl = None if c["seqlens"] is None else c["seqlens"][b]
        vis = ref.visible(np.arange(N), N, c["causal"], sl, c["block_mask"], c["mask_block"])
        for h in range(H):
            P = O[b, h]
            assert np.all(P >= 0)
            assert np.all(P[~vis] == 0)
            live = vis.any(axis=1)
            np.testing.assert_allclose(P[live].sum(axis=1), 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("kind", MASK_KINDS)
def test_constant_values(kind):
    c = _case(kind)
    v = np.full_like(c["v"], 2.5)
    O, _ = _fwd(c, v=v)
    live = np.isfinite(_fwd(c)[1])
    np.testing.assert_allclose(O[live], 2.5, rtol=0, atol=1e-13)
    assert np.all(O[~live] == 0)


@pytest.mark.parametrize("kind", MASK_KINDS)
def test_zero_queries_give_mean_of_visible_values(kind):
    c = _case(kind)
    B, H, N, d = c["q"].shape
    O, L = _fwd(c, q=np.zeros_like(c["q"]))
    for b in range(B):
        sl = None if c["seqlens"] is None else c["seqlens"][b]
        vis = ref.visible(np.arange(N), N, c["causal"], sl, c["block_mask"], c["mask_block"])
        for h in range(H):
            for i in range(N):
                n = vis[i].sum()
                if n == 0:
                    assert L[b, h, i] == -np.inf and np.all(O[b, h, i] == 0)
                    continue
                np.testing.assert_allclose(O[b, h, i], c["v"][b, h][vis[i]].mean(axis=0),
                                           rtol=0, atol=1e-13)
                assert abs(L[b, h, i] - math.log(n)) < 1e-13


def test_causal_first_row_and_single_key():
    c = _case("causal")
    O, L = _fwd(c)
    s00 = c["scale"] * np.einsum("bhd,bhd->bh", c["q"][:, :, 0], c["k"][:, :, 0])
    np.testing.assert_allclose(O[:, :, 0], c["v"][:, :, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(L[:, :, 0], s00, rtol=0, atol=1e-14)
    # one visible key for every row: non-causal with key length 1
    c2 = _case("none")
    O2, L2 = _fwd(c2, seqlens=np.ones(1, np.int32))
    s = c2["scale"] * np.einsum("bhnd,bhd->bhn", c2["q"], c2["k"][:, :, 0])
    np.testing.assert_allclose(O2, np.broadcast_to(c2["v"][:, :, :1], O2.shape), rtol=0,
                               atol=1e-14)
    np.testing.assert_allclose(L2, s, rtol=0, atol=1e-14)


@pytest.mark.parametrize("kind", MASK_KINDS)
def test_row_shift_moves_L_only(kind):
    """Adding c_i to every score of row i (via an extra feature) leaves P, hence
    O, unchanged and shifts L_i by c_i."""
    c = _case(kind)
    B, H, N, d = c["q"].shape
    rng = np.random.default_rng(7)
    shift = rng.uniform(-50, 50, size=(B, H, N))
    q2 = np.concatenate([c["q"], (shift / c["scale"])[..., None]], axis=-1)
    k2 = np.concatenate([c["k"], np.ones((B, H, N, 1))], axis=-1)
    O1, L1 = _fwd(c)
    O2, L2 = _fwd(c, q=q2, k=k2)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
    live = np.isfinite(L1)
    np.testing.assert_allclose(L2[live], L1[live] + shift[live], rtol=0, atol=1e-11)


def test_key_permutation_invariance():
    c = _case("none", N=16)
    perm = np.random.default_rng(3).permutation(16)
    O1, L1 = _fwd(c)
    O2, L2 = _fwd(c, k=c["k"][:, :, perm], v=c["v"][:, :, perm])
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L2, L1, rtol=0, atol=1e-13)


@pytest.mark.parametrize("kind", MASK_KINDS)
@pytest.mark.parametrize("block", [1, 3, 7, 64])
def test_online_softmax_equals_two_pass(kind, block):
    c = _case(kind, N=20, mask_block=4)
    O1, L1 = _fwd(c)
    O2, L2 = ref.forward_online(c["q"], c["k"], c["v"], c["scale"], c["causal"], c["seqlens"],
                                c["block_mask"], c["mask_block"], key_block=block)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
    live = np.isfinite(L1)
    assert np.array_equal(live, np.isfinite(L2))
    np.testing.assert_allclose(L2[live], L1[live], rtol=0, atol=1e-12)


@pytest.mark.parametrize("big", [20000.0, -20000.0])
def test_safe_softmax_huge_equal_scores(big):
    """All scores equal to +-20000 (the overflow / underflow cases of the
    llm-deploy note): P is uniform and everything stays finite."""
    N, d = 8, 4
    q = np.full((1, 1, N, d), 1.0)
    k = np.full((1, 1, N, d), big / d)
    rng = np.random.default_rng(0)
    v = rng.standard_normal((1, 1, N, d))
    O, L = ref.forward(q, k, v, 1.0)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0].mean(0), (N, d)), atol=1e-12)
    np.testing.assert_allclose(L, big + math.log(N), rtol=1e-15)


def test_safe_softmax_mixed_huge_scores():
    """One key at +20000 and the rest at -20000: P is one-hot on that key."""
    N, d = 6, 1
    q = np.ones((1, 1, N, d))
    kk = np.full(N, -20000.0)
    kk[2] = 20000.0
    k = kk.reshape(1, 1, N, 1)
    v = np.arange(N, dtype=float).reshape(1, 1, N, 1)
    O, L = ref.forward(q, k, v, 1.0)
    np.testing.assert_allclose(O.ravel(), 2.0, atol=0)
    np.testing.assert_allclose(L.ravel(), 20000.0, rtol=1e-15)


def test_all_ones_block_mask_and_full_length_equal_dense():
    c = _case("none", N=16)
    O1, L1 = _fwd(c)
    O2, L2 = _fwd(c, block_mask=np.ones((4, 4), np.uint8))
    O3, L3 = _fwd(c, seqlens=np.full(1, 16, np.int32))
    for O, L in [(O2, L2), (O3, L3)]:
        np.testing.assert_array_equal(O, O1)
        np.testing.assert_array_equal(L, L1)


@pytest.mark.parametrize("kind", MASK_KINDS)
def test_L_bounds(kind):
    c = _case(kind)
    B, H, N, d = c["q"].shape
    _, L = _fwd(c)
    for b in range(B):
        sl = None if c["seqlens"] is None else c["seqlens"][b]
        vis = ref.visible(np.arange(N), N, c["causal"], sl, c["block_mask"], c["mask_block"])
        for h in range(H):
            s = c["scale"] * c["q"][b, h] @ c["k"][b, h].T
            for i in range(N):
                if not vis[i].any():
                    continue
                mx = s[i][vis[i]].max()
                assert mx - 1e-12 <= L[b, h, i] <= mx + math.log(vis[i].sum()) + 1e-12


def test_fully_masked_rows():
    """A query row with no visible key: O = 0, L = -inf, and it adds nothing to
    dK / dV (same as zeroing its dO)."""
    c = _case("none", N=8, mask_block=4)
    bm = np.array([[0, 0], [1, 1]], np.uint8)   # rows 0..3 see nothing
    O, L = _fwd(c, block_mask=bm)
    assert np.all(O[:, :, :4] == 0) and np.all(L[:, :, :4] == -np.inf)
    assert np.all(np.isfinite(L[:, :, 4:]))
    dq, dk, dv = _bwd(c, block_mask=bm)
    do2 = c["do"].copy()
    do2[:, :, :4] = 0
    _, dk2, dv2 = _bwd(c, block_mask=bm, do=do2)
    assert np.all(dq[:, :, :4] == 0)
    np.testing.assert_allclose(dk, dk2, atol=1e-14)
    np.testing.assert_allclose(dv, dv2, atol=1e-14)
    # key length 0 for a sequence: every row fully masked
    O3, L3 = _fwd(c, seqlens=np.zeros(1, np.int32))
    assert np.all(O3 == 0) and np.all(L3 == -np.inf)


def test_masked_keys_get_zero_gradient():
    c = _case("padded", N=12)
    dq, dk, dv = _bwd(c)
    for b in range(c["q"].shape[0]):
        n = c["seqlens"][b]
        assert np.all(dk[b, :, n:] == 0) and np.all(dv[b, :, n:] == 0)


# ------------------------------------------------------------ gradient pins

@pytest.mark.parametrize("kind", MASK_KINDS)
def test_gradients_match_central_finite_differences(kind):
    c = _case(kind, B=1, H=2, N=12, d=4, mask_block=4)
    dq, dk, dv = _bwd(c)

    def f(**over):
        O, _ = _fwd(c, **over)
        return float((c["do"] * O).sum())

    h = 1e-6
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        x = c[name]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy()
            xp[idx] += h
            xm = x.copy()
            xm[idx] -= h
            num[idx] = (f(**{name: xp}) - f(**{name: xm})) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg=f"d{name} ({kind})")


@pytest.mark.parametrize("kind", MASK_KINDS)
def test_gradient_sum_identities(kind):
    """Softmax rows are invariant to adding a constant to all keys' scores, so
    sum_j dK_j = 0; and sum_j P_ij = 1 gives sum_j dV_j = sum over live rows of dO_i."""
    c = _case(kind, N=16)
    _, L = _fwd(c)
    dq, dk, dv = _bwd(c)
    live = np.isfinite(L)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    exp_dv = np.where(live[..., None], c["do"], 0.0).sum(axis=2)
    np.testing.assert_allclose(dv.sum(axis=2), exp_dv, atol=1e-12)


# --------------------------------------------------------- sampled variants

@pytest.mark.parametrize("kind", MASK_KINDS)
def test_sampled_rows_match_full(kind):
    c = _case(kind, B=2, H=2, N=24, mask_block=8)
    rng = np.random.default_rng(11)
    rows = wl.sample_rows(rng, 2, 2, 24, 7)
    O, L = _fwd(c)
    Os, Ls = ref.forward(c["q"], c["k"], c["v"], c["scale"], c["causal"], c["seqlens"],
                         c["block_mask"], c["mask_block"], rows=rows)
    dq, _, _ = _bwd(c)
    dqs, dks, dvs = ref.backward(c["q"], c["k"], c["v"], c["do"], c["scale"], c["causal"],
                                 c["seqlens"], c["block_mask"], c["mask_block"], rows=rows)
    do_r = np.zeros_like(c["do"])
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(Os[b, h], O[b, h, rows[b, h]], atol=1e-14)
            np.testing.assert_allclose(Ls[b, h], L[b, h, rows[b, h]], atol=1e-14)
            np.testing.assert_allclose(dqs[b, h], dq[b, h, rows[b, h]], atol=1e-13)
            do_r[b, h, rows[b, h]] = c["do"][b, h, rows[b, h]]
    _, dk_r, dv_r = _bwd(c, do=do_r)
    np.testing.assert_allclose(dks, dk_r, atol=1e-13)
    np.testing.assert_allclose(dvs, dv_r, atol=1e-13)


def test_pair_count_closed_forms():
    N = 40
    assert ref.visible_pair_count(N) == N * N
    assert ref.visible_pair_count(N, causal=True) == N * (N + 1) // 2
    sl = np.array([3, 17, 40], np.int32)
    assert ref.visible_pair_count(N, seqlens=sl, B=3) == N * int(sl.sum())
    bm = wl.draw_block_mask(np.random.default_rng(1), N, 0.3, 8)
    assert ref.visible_pair_count(N, block_mask=bm, mask_block=8) == int(bm.sum()) * 64


# ------------------------------------------------------ library cross-check

@pytest.mark.parametrize("kind", MASK_KINDS)
def test_matches_torch_float64_sdpa_and_autograd(kind):
    torch = pytest.importorskip("torch")
    c = _case(kind, B=2, H=3, N=16, d=8, mask_block=4)
    _, L = _fwd(c)
    if not np.all(np.isfinite(L)):
        pytest.skip("library routine yields NaN on fully masked rows")
    B, H, N, d = c["q"].shape
    mask = np.zeros((B, 1, N, N), bool)
    for b in range(B):
        sl = None if c["seqlens"] is None else c["seqlens"][b]
        mask[b, 0] = ref.visible(np.arange(N), N, c["causal"], sl, c["block_mask"],
                                 c["mask_block"])
    tq, tk, tv = (torch.tensor(c[n], dtype=torch.float64, requires_grad=True)
                  for n in ("q", "k", "v"))
    tm = torch.tensor(mask)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm,
                                                           scale=c["scale"])
    out.backward(torch.tensor(c["do"]))
    lse = torch.logsumexp((c["scale"] * tq @ tk.transpose(-1, -2)).masked_fill(~tm, -math.inf),
                          dim=-1)
    O, L = _fwd(c)
    dq, dk, dv = _bwd(c)
    np.testing.assert_allclose(O, out.detach().numpy(), atol=1e-13)
    np.testing.assert_allclose(L, lse.detach().numpy(), atol=1e-13)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


# ------------------------------------------------- N_q != N_k (cached keys)

def _rect(Nq, Nk, kind, seed=0, d=4, B=1, H=2, mask_block=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Nq, d))
    k, v = (rng.standard_normal((B, H, Nk, d)) for _ in range(2))
    do = rng.standard_normal((B, H, Nq, d))
    causal = kind in ("causal", "causal_padded_block")
    seqlens = None
    block = None
    if kind in ("padded", "causal_padded_block"):
        seqlens = rng.integers(max(1, Nk // 2), Nk + 1, size=B).astype(np.int32)
    if kind in ("block", "causal_padded_block"):
        tq, tk = -(-Nq // mask_block), -(-Nk // mask_block)
        block = (rng.random((tq, tk)) < 0.6).astype(np.uint8)
    return dict(q=q, k=k, v=v, do=do, scale=0.7, causal=causal, seqlens=seqlens,
                block_mask=block, mask_block=mask_block)


def _mk(c):
    return dict(causal=c["causal"], seqlens=c["seqlens"], block_mask=c["block_mask"],
                mask_block=c["mask_block"])


@pytest.mark.parametrize("Nq", [1, 3, 7])
def test_cached_keys_equal_the_suffix_of_the_square_problem(Nq):
    """Causal with N_q < N_k: the N_q queries are the last positions of a
    sequence of N_k, so their outputs are the last rows of the square causal
    problem; gradients likewise, with dO zero on the earlier rows."""
    Nk = 11
    rng = np.random.default_rng(Nq)
    qf, k, v, dof = (rng.standard_normal((1, 2, Nk, 5)) for _ in range(4))
    dof[:, :, :Nk - Nq] = 0.0
    Of, Lf = ref.forward(qf, k, v, 0.6, causal=True)
    O, L = ref.forward(qf[:, :, Nk - Nq:], k, v, 0.6, causal=True)
    np.testing.assert_allclose(O, Of[:, :, Nk - Nq:], rtol=0, atol=1e-14)
    np.testing.assert_allclose(L, Lf[:, :, Nk - Nq:], rtol=0, atol=1e-14)
    gf = ref.backward(qf, k, v, dof, 0.6, causal=True)
    g = ref.backward(qf[:, :, Nk - Nq:], k, v, dof[:, :, Nk - Nq:], 0.6, causal=True)
    np.testing.assert_allclose(g[0], gf[0][:, :, Nk - Nq:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(g[1], gf[1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(g[2], gf[2], rtol=0, atol=1e-13)


def test_decode_row_sees_every_key():
    c = _rect(1, 9, "none", seed=3)
    O1, L1 = ref.forward(c["q"], c["k"], c["v"], c["scale"], causal=True)
    O0, L0 = ref.forward(c["q"], c["k"], c["v"], c["scale"], causal=False)
    np.testing.assert_array_equal(O1, O0)
    np.testing.assert_array_equal(L1, L0)


def test_more_queries_than_keys_leaves_leading_rows_dead():
    """Causal with N_q > N_k: query i sees keys j <= i - (N_q - N_k), so the
    first N_q - N_k rows see nothing and the rest are the square problem."""
    Nq, Nk = 9, 5
    c = _rect(Nq, Nk, "none", seed=4)
    O, L = ref.forward(c["q"], c["k"], c["v"], c["scale"], causal=True)
    assert np.all(O[:, :, :Nq - Nk] == 0) and np.all(np.isneginf(L[:, :, :Nq - Nk]))
    Os, Ls = ref.forward(c["q"][:, :, Nq - Nk:], c["k"], c["v"], c["scale"], causal=True)
    np.testing.assert_allclose(O[:, :, Nq - Nk:], Os, rtol=0, atol=1e-15)
    np.testing.assert_allclose(L[:, :, Nq - Nk:], Ls, rtol=0, atol=1e-15)
    dq, dk, dv = ref.backward(c["q"], c["k"], c["v"], c["do"], c["scale"], causal=True)
    assert np.all(dq[:, :, :Nq - Nk] == 0)


@pytest.mark.parametrize("Nq,Nk", [(5, 9), (9, 5)])
@pytest.mark.parametrize("kind", MASK_KINDS)
def test_rectangular_online_and_finite_differences(Nq, Nk, kind):
    c = _rect(Nq, Nk, kind, seed=Nq * 10 + Nk)
    kw = _mk(c)
    O, L = ref.forward(c["q"], c["k"], c["v"], c["scale"], **kw)
    O2, L2 = ref.forward_online(c["q"], c["k"], c["v"], c["scale"], key_block=3, **kw)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
    live = np.isfinite(L)
    np.testing.assert_allclose(L2[live], L[live], rtol=0, atol=1e-12)
    dq, dk, dv = ref.backward(c["q"], c["k"], c["v"], c["do"], c["scale"], **kw)
    assert dq.shape == c["q"].shape and dk.shape == c["k"].shape

    def f(q, k, v):
        return float((c["do"] * ref.forward(q, k, v, c["scale"], **kw)[0]).sum())

    h = 1e-6
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        x = {n: c[n].copy() for n in ("q", "k", "v")}
        num = np.zeros_like(g)
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x[name][idx] += h
            fp = f(x["q"], x["k"], x["v"])
            x[name][idx] -= 2 * h
            fm = f(x["q"], x["k"], x["v"])
            x[name][idx] += h
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_rectangular_pair_count():
    # causal, N_q = 3 cached after 5 keys: rows see 6, 7, 8 keys
    assert ref.visible_pair_count(3, causal=True, N_k=8) == 6 + 7 + 8
    # N_q = 8 over N_k = 3: rows 5, 6, 7 see 1, 2, 3 keys
    assert ref.visible_pair_count(8, causal=True, N_k=3) == 1 + 2 + 3
