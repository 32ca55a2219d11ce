"""Pins for the dropout oracle (oracle/dropout_ref.py): the generator against
its published known-answer vectors, the reduction to plain attention at p = 0,
the statistics of the keep decisions, central finite differences of the
gradients with the mask held fixed, and unbiasedness over seeds."""
import os

import numpy as np
import pytest

from oracle import attention_ref as ref
from oracle import dropout_ref as dref
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat_rows():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x, 16) for x in line.split()])
    return rows


@pytest.mark.parametrize("row", _kat_rows())
def test_philox_known_answers(row):
    ctr, key, out = row[:4], row[4:6], row[6:]
    got = dref.philox4x32(np.array(ctr), np.array(key))
    assert [int(x) for x in got] == out


def test_philox_is_vectorised_elementwise():
    rng = np.random.default_rng(3)
    ctr = rng.integers(0, 2**32, size=(5, 7, 4), dtype=np.uint64)
    key = np.array([0x12345678, 0x9abcdef0])
    got = dref.philox4x32(ctr, key)
    for idx in [(0, 0), (4, 6), (2, 3)]:
        one = dref.philox4x32(ctr[idx], key)
        assert np.array_equal(got[idx], one)


def test_threshold_reading():
    assert dref.keep_threshold(0.0) == 256
    assert dref.keep_threshold(0.5) == 128
    assert dref.keep_threshold(0.1) == 230          # 230.4 rounds down
    assert dref.keep_threshold(1 - 100.5 / 256) == 101  # a tie rounds up
    with pytest.raises(ValueError):
        dref.keep_threshold(1.0)
    with pytest.raises(ValueError):
        dref.keep_threshold(0.999)


def test_uniform_bytes_follow_the_counter_layout():
    """u_ij is byte (j mod 4) of word (i mod 4) of the call whose counter is
    (j div 4, i div 4, bh, offset): evaluated pair by pair, one call each."""
    seed, offset, bh = 0x0123456789ABCDEF, 7, 5
    rows = np.array([0, 1, 2, 3, 6, 37, 100])
    u = dref.uniform_bytes(rows, 23, bh, seed, offset)
    key = np.array([seed & 0xFFFFFFFF, seed >> 32])
    for r, i in enumerate(rows):
        for j in range(23):
            w = dref.philox4x32(np.array([j // 4, i // 4, bh, offset]), key)
            assert u[r, j] == (int(w[i % 4]) >> (8 * (j % 4))) & 0xFF


def test_keep_rate_and_byte_uniformity():
    rows = np.arange(512)
    u = dref.uniform_bytes(rows, 512, 3, 2024, 0).astype(np.int64)
    n = u.size
    counts = np.bincount(u.ravel(), minlength=256)
    chi2 = float(((counts - n / 256) ** 2 / (n / 256)).sum())
    assert abs(chi2 - 255) < 6 * np.sqrt(2 * 255), chi2
    for p in (0.1, 0.25, 0.5, 0.9):
        t = dref.keep_threshold(p)
        frac = float((u < t).mean())
        sd = np.sqrt(t / 256 * (1 - t / 256) / n)
        assert abs(frac - t / 256) < 5 * sd, (p, frac)
    # different heads, offsets and seeds give different masks
    assert not np.array_equal(u, dref.uniform_bytes(rows, 512, 4, 2024, 0))
    assert not np.array_equal(u, dref.uniform_bytes(rows, 512, 3, 2024, 1))
    assert not np.array_equal(u, dref.uniform_bytes(rows, 512, 3, 2025, 0))


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


def _mask_kw(c):
    return dict(causal=c["causal"], seqlens=c["seqlens"], block_mask=c["block_mask"],
                mask_block=c["mask_block"])


@pytest.mark.parametrize("kind", MASK_KINDS)
def test_zero_probability_is_plain_attention(kind):
    c = _case(kind, B=2, N=20)
    O0, L0 = ref.forward(c["q"], c["k"], c["v"], c["scale"], **_mask_kw(c))
    O1, L1 = dref.forward(c["q"], c["k"], c["v"], c["scale"], 0.0, 99, **_mask_kw(c))
    np.testing.assert_allclose(O1, O0, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(L1, L0)
    g0 = ref.backward(c["q"], c["k"], c["v"], c["do"], c["scale"], **_mask_kw(c))
    g1 = dref.backward(c["q"], c["k"], c["v"], c["do"], c["scale"], 0.0, 99, **_mask_kw(c))
    for a, b in zip(g1, g0):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_lse_ignores_dropout_and_dropped_pairs_carry_nothing():
    c = _case("none", N=16)
    O0, L0 = ref.forward(c["q"], c["k"], c["v"], c["scale"])
    O1, L1 = dref.forward(c["q"], c["k"], c["v"], c["scale"], 0.4, 5)
    np.testing.assert_array_equal(L1, L0)
    # V nonzero only at one key: O_i is s P_ij v_j if (i, j) is kept, else 0
    v = np.zeros_like(c["v"])
    v[:, :, 9, :] = 1.0
    O2, _ = dref.forward(c["q"], c["k"], v, c["scale"], 0.4, 5)
    for h in range(2):
        z = dref.keep_mask(np.arange(16), 16, h, 0.4, 5, 0)[:, 9]
        assert np.all((O2[0, h, :, 0] != 0) == z)


@pytest.mark.parametrize("kind", MASK_KINDS)
def test_gradients_match_finite_differences(kind):
    c = _case(kind)
    p, seed = 0.3, 11
    kw = _mask_kw(c)
    dq, dk, dv = dref.backward(c["q"], c["k"], c["v"], c["do"], c["scale"], p, seed, **kw)

    def f(q, k, v):
        O, _ = dref.forward(q, k, v, c["scale"], p, seed, **kw)
        return float((c["do"] * O).sum())

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


def test_output_is_unbiased_over_seeds():
    c = _case("causal", N=8, d=3, seed=4)
    O0, _ = ref.forward(c["q"], c["k"], c["v"], c["scale"], causal=True)
    outs = np.stack([dref.forward(c["q"], c["k"], c["v"], c["scale"], 0.5, s, causal=True)[0]
                     for s in range(1500)])
    mean = outs.mean(axis=0)
    se = outs.std(axis=0) / np.sqrt(outs.shape[0])
    # row 0 sees one key: its output is 0 or 2 v_0, exactly unbiased too
    assert np.all(np.abs(mean - O0) <= 6 * se + 1e-12)


def test_sampled_rows_equal_full_rows():
    c = _case("causal_padded_block", B=2, N=20)
    kw = _mask_kw(c)
    O, L = dref.forward(c["q"], c["k"], c["v"], c["scale"], 0.2, 8, 3, **kw)
    rows = np.array([[[1, 7, 19], [0, 4, 12]], [[2, 3, 18], [5, 6, 11]]])
    Os, Ls = dref.forward(c["q"], c["k"], c["v"], c["scale"], 0.2, 8, 3, rows=rows, **kw)
    for b in range(2):
        for h in range(2):
            np.testing.assert_array_equal(Os[b, h], O[b, h, rows[b, h]])
            np.testing.assert_array_equal(Ls[b, h], L[b, h, rows[b, h]])
    dq, _, _ = dref.backward(c["q"], c["k"], c["v"], c["do"], c["scale"], 0.2, 8, 3, **kw)
    dqs, _, _ = dref.backward(c["q"], c["k"], c["v"], c["do"], c["scale"], 0.2, 8, 3,
                              rows=rows, **kw)
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(dqs[b, h], dq[b, h, rows[b, h]], rtol=0, atol=1e-14)
