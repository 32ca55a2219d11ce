"""Seeded input generator: determinism, bf16 rounding, mask and sample shapes."""
import numpy as np
import pytest

import workloads as wl


def test_bf16_rounding_matches_library_rne():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0],
                                 np.float32)])
    ours = wl.round_to_bf16(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), lib.view(np.uint32))
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert wl.round_to_bf16(np.array([1.0 + 2 ** -8], np.float32))[0] == 1.0
    assert wl.round_to_bf16(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 1.0 + 2 ** -6


def test_bf16_bits_roundtrip():
    x = wl.round_to_bf16(np.random.default_rng(1).standard_normal(1000).astype(np.float32))
    b = wl.bf16_bits(x)
    back = (b.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(back, x)
    with pytest.raises(ValueError):
        wl.bf16_bits(np.array([1.0 + 2 ** -20], np.float32))


def test_inputs_are_deterministic_and_seeded():
    w = wl.WORKLOADS["bertl_padded_b16h16n512"]
    a = wl.make_inputs(w)
    b = wl.make_inputs(w)
    for key in ("q", "k", "v", "do", "seqlens"):
        np.testing.assert_array_equal(a[key], b[key])
    c = wl.make_inputs(w, seed=99)
    assert not np.array_equal(a["q"], c["q"])
    assert a["seqlens"].min() >= 256 and a["seqlens"].max() <= 512
    assert a["q"].shape == (16, 16, 512, 64)
    assert np.all(wl.round_to_bf16(a["q"]) == a["q"])


def test_block_mask_diagonal_and_density():
    rng = np.random.default_rng(5)
    m = wl.draw_block_mask(rng, 65536, 1 / 16)
    assert m.shape == (512, 512) and m.dtype == np.uint8
    assert np.all(np.diag(m) == 1)
    off = m[~np.eye(512, dtype=bool)]
    assert abs(off.mean() - 1 / 16) < 0.01


def test_sample_rows_unique_sorted():
    rows = wl.sample_rows(np.random.default_rng(2), 2, 3, 100, 10)
    assert rows.shape == (2, 3, 10)
    for r in rows.reshape(-1, 10):
        assert len(set(r.tolist())) == 10 and np.all(np.diff(r) > 0)


def test_small_config_values():
    w = wl.WORKLOADS["single_head_f32_n128"]
    a = wl.make_inputs(w)
    assert a["q"].dtype == np.float32 and a["q"].shape == (1, 1, 128, 64)
    # fp32 workload is not bf16-rounded
    assert not np.all(wl.round_to_bf16(a["q"]) == a["q"])
