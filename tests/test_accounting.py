"""The bench's FLOP accounting: closed-form pair counts against a brute-force
count over the oracle's materialised mask, and the single-GPU guard."""
import numpy as np
import pytest

import bench
import workloads as wl
from oracle import attention_ref as ref


@pytest.mark.parametrize("N,causal,seqlens,p", [
    (300, True, [100, 300, 0], 0.4),
    (256, False, None, 0.3),
    (200, True, None, None),
    (130, False, [5, 130], None),
    (384, True, [384, 200], 0.5),
    (1, False, None, None),
])
def test_pairs_match_brute_force(N, causal, seqlens, p):
    rng = np.random.default_rng(N)
    bm = wl.draw_block_mask(rng, N, p) if p else None
    B = 1 if seqlens is None else len(seqlens)
    sl = None if seqlens is None else np.array(seqlens, np.int32)
    got = bench.visible_pairs(N, 3, causal, sl, bm, 128, B)
    want = 3 * ref.visible_pair_count(N, causal, sl, bm, 128, B)
    assert got == want


def test_workload_pair_counts():
    w = wl.WORKLOADS["gpt2s_causal_b8h12n1024"]
    assert bench.visible_pairs(w.N, w.H, True, None, None, 128, w.B) == 50_380_800
    w = wl.WORKLOADS["long_causal_b1h16n16384"]
    assert bench.visible_pairs(w.N, w.H, True, None, None, 128, w.B) == 2_147_614_720
    w = wl.WORKLOADS["blocksparse_b1h8n65536"]
    bm = wl.draw_block_mask(np.random.default_rng(0), w.N, 1 / 16)
    assert bench.visible_pairs(w.N, w.H, False, None, bm, 128, 1) == 8 * int(bm.sum()) * 128 * 128


def test_kernel_bytes():
    kb = bench.kernel_bytes(8, 12, 1024, 64, 2, None)
    t = 8 * 12 * 1024 * 64 * 2
    row = 8 * 12 * 1024 * 4
    assert kb["fa_fwd"] == 4 * t + row
    assert kb["fa_bwd"] == 8 * t + 3 * row  # L read, D written and read
    kb2 = bench.kernel_bytes(2, 1, 100, 64, 2, np.array([50, 100]))
    assert kb2["fa_fwd"] == 2 * (2 * 100 * 64 * 2) + 2 * (150 * 64 * 2) + 2 * 100 * 4


def test_kernel_flops_are_the_method():
    kf = bench.kernel_flops(64, 1000)
    assert kf["fa_fwd"] == 4 * 64 * 1000
    assert kf["fa_bwd"] == 10 * 64 * 1000


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_io_sweep_model_and_dispatch_mapping():
    import bench
    m = bench.sweep_model(1024, 128, H=16, d=64)
    t = 1024 * 64 * 2
    assert m["compulsory"] == 16 * (4 * t + 4 * 1024)
    assert m["kv_streamed"] == 16 * 8 * 2 * t          # 8 query tiles of 128 rows
    assert bench.sweep_model(1024, 64)["kv_streamed"] == 2 * m["kv_streamed"]
    assert bench.sweep_model(1024, 256)["kv_streamed"] * 2 == m["kv_streamed"]
    # every configuration's launch shape is distinct, whether or not the
    # 128-row tiles split their keys over 3 groups of waves
    for groups128 in (1, 3):
        shapes, launches = {}, []
        for N in bench.SWEEP_N:
            for bq in bench.SWEEP_BQ:
                threads = 2 * bq * (groups128 if bq == 128 else 1)  # 64 lanes per wave
                wgs = (N // bq) * bench.SWEEP_H
                assert (wgs, threads) not in shapes
                shapes[(wgs, threads)] = (N, bq)
                launches.append((dict(wg=threads, grid=wgs * threads), (N, bq)))
        for d, cfg in launches:                       # Grid_Size counts work-items
            assert bench._sweep_config(d, shapes) == cfg


@pytest.mark.parametrize("N,Nk,causal,seqlens,p", [
    (100, 300, True, None, None),
    (300, 100, True, None, None),
    (130, 500, True, [400, 20], 0.5),
    (500, 130, True, [130, 60], 0.5),
    (200, 450, False, [450, 300], 0.4),
])
def test_rectangular_pairs_match_brute_force(N, Nk, causal, seqlens, p):
    rng = np.random.default_rng(N + Nk)
    bm = None
    if p:
        bm = (rng.random((-(-N // 128), -(-Nk // 128))) < p).astype(np.uint8)
    B = 1 if seqlens is None else len(seqlens)
    sl = None if seqlens is None else np.array(seqlens, np.int32)
    got = bench.visible_pairs(N, 2, causal, sl, bm, 128, B, Nk=Nk)
    want = 2 * ref.visible_pair_count(N, causal, sl, bm, 128, B, N_k=Nk)
    assert got == want


def test_rectangular_kernel_bytes():
    kb = bench.kernel_bytes(1, 2, 100, 64, 2, None, Nk=300)
    tq, tk = 2 * 100 * 64 * 2, 2 * 300 * 64 * 2
    assert kb["fa_fwd"] == 2 * tq + 2 * tk + 2 * 100 * 4
    assert kb["fa_bwd"] == 4 * tq + 4 * tk + 3 * 2 * 100 * 4


def test_pipe_metrics_formulas():
    # A dispatch of 1000 GPU-active cycles on 256 CUs x 4 SIMDs in which every
    # SIMD has its matrix core busy for 400 cycles and a vector instruction
    # executing for 600 (counted in quad-cycles per CU: 4 SIMDs x 600 / 4).
    # GRBM_GUI_ACTIVE comes summed over the 8 XCDs.
    c = dict(GRBM_GUI_ACTIVE=8 * 1000.0, SQ_VALU_MFMA_BUSY_CYCLES=1024 * 400.0,
             SQ_ACTIVE_INST_VALU=256 * 600.0, SQ_BUSY_CU_CYCLES=256 * 1000.0,
             SQ_LDS_BANK_CONFLICT=5.0, SQ_LDS_IDX_ACTIVE=100.0,
             SQ_INSTS_VALU_TRANS_F32=300.0, SQ_INSTS_MFMA=1200.0)
    m = bench.pipe_metrics(c)
    assert m["mfma_busy"] == pytest.approx(0.4)
    assert m["valu_busy"] == pytest.approx(0.6)
    assert m["cu_busy"] == pytest.approx(1.0)
    assert m["lds_conflict"] == pytest.approx(0.05)
    assert m["trans_per_mfma"] == pytest.approx(0.25)
    assert m["gui_cycles"] == pytest.approx(1000.0)
    assert len(bench.PIPE_COUNTERS) == 8
    assert sum(n.startswith("SQ_") for n in bench.PIPE_COUNTERS) <= 8
    assert sum(n.startswith("GRBM_") for n in bench.PIPE_COUNTERS) <= 2


def test_launch_durations_of_sampled_steps():
    class Ev:
        def __init__(self, t):
            self.t = t

        def elapsed_time(self, other):
            return other.t - self.t

    # two sampled steps: (fwd 2 ms, bwd 5 ms) and (3, 4)
    samples = [[Ev(1.0), Ev(3.0), Ev(8.0)], [Ev(20.0), Ev(23.0), Ev(27.0)]]
    d = bench.launch_durations(samples, ("fwd", "bwd"))
    assert d == {"fwd": [2.0, 3.0], "bwd": [5.0, 4.0]}
    # forward-only steps: a start and one launch
    d = bench.launch_durations([[Ev(0.0), Ev(2.0)], [Ev(5.0), Ev(8.0)]], ("fwd",))
    assert d == {"fwd": [2.0, 3.0]}


@pytest.mark.parametrize("N,Nk,causal,seqlens,p", [
    (300, 300, True, [100, 300], 0.4),
    (512, 512, False, None, 0.3),
    (200, 700, True, None, None),
    (260, 130, True, [5, 130], 0.5),
    (384, 384, False, [384, 200], None),
])
def test_sampled_pairs_match_brute_force(N, Nk, causal, seqlens, p):
    rng = np.random.default_rng(N + Nk)
    bm = None
    if p:
        bm = (rng.random((-(-N // 128), -(-Nk // 128))) < p).astype(np.uint8)
    B, H = (1 if seqlens is None else len(seqlens)), 3
    sl = None if seqlens is None else np.array(seqlens, np.int32)
    rows = wl.sample_rows(rng, B, H, N, min(N, 37))
    want = 0
    for b in range(B):
        for h in range(H):
            vis = ref.visible(rows[b, h], Nk, causal, None if sl is None else sl[b], bm, 128, N)
            want += int(vis.sum())
    assert bench.sampled_pairs(rows, N, causal, sl, bm, 128, Nk=Nk) == want
