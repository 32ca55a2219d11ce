#!/usr/bin/env python3
"""Attention throughput on one MI355X.

One step = the whole hot path on one batch: fa_fwd (scores, mask, online
softmax, O and L) followed by fa_bwd (D, dQ, dK, dV recomputed from L), one
kernel launch each.
Prints one JSON line with forward+backward TFLOP/s (the value), forward
TFLOP/s, both as fractions of the bf16 dense MFMA peak, a roofline entry for
the dominant kernel and the fp64 CPU oracle timed on the host as a baseline.

FLOP convention (algorithmic work over visible (query, key) pairs; masked-out
tiles are never credited): forward 4*d*pairs, backward 10*d*pairs.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--dropout P]
                    [--cpu-baseline off]

--dropout P times fa_fwd_dropout / fa_bwd_dropout (keep mask regenerated in
every kernel from Philox4x32-10) on the same workload and FLOP count.

HBM traffic of the dominant kernel comes from rocprofv3 counter runs kept in
profiles/hbm_traffic_<workload>.json (written by --pmc-summary from a
FETCH_SIZE run and a WRITE_SIZE run of this script, scaled by the same
counters read on a plain copy of known size, --mode copy); it is reported
only while the kernel's sources still hash to the value recorded there.

After the timed steps, --cold-reps launches of each kernel are timed again,
each after a 1 GiB write that evicts L2 and the Infinity Cache (cold-cache
medians, reported beside the warm back-to-back figures).  --pipe-summary
turns a rocprofv3 run of SQ/GRBM counters into profiles/pipe_counters_<key>.md
(MFMA and VALU busy fractions, transcendental instructions, LDS bank
conflicts).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "attention TFLOP/s (fwd, fwd+bwd) and % of MI355X bf16 MFMA peak"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # dense MFMA bf16; fp32 vector/matrix
PEAK_HBM_GBS = 8000.0
FLUSH_BYTES = 1 << 30   # cold-cache runs: larger than L2 (8 x 4 MB) + Infinity Cache (256 MB)
# Counters of one --pmc pass for --pipe-summary (7 SQ + 1 GRBM, within the
# per-pass limits of the SQ and GRBM blocks).
PIPE_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU_TRANS_F32",
                 "SQ_INSTS_MFMA", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
                 "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")
DEFAULT_WORKLOAD = "blocksparse_b1h8n65536"


# --------------------------------------------------------------- accounting

def visible_pairs(N: int, H: int, causal: bool, seqlens, block_mask, mask_block: int = 128,
                  B: int = 1, Nk=None) -> int:
    """Number of visible (query, key) pairs summed over batch and heads: N
    queries, Nk keys (default N), causal key j visible to query i iff
    j <= i + Nk - N."""
    Nk = N if Nk is None else Nk
    off = Nk - N
    lens = [Nk] * B if seqlens is None else [int(min(max(s, 0), Nk)) for s in seqlens]
    total = 0
    for L in lens:
        if block_mask is None:
            if causal:
                i = np.arange(N, dtype=np.int64)
                total += int(np.clip(np.minimum(i + 1 + off, L), 0, None).sum())
            else:
                total += N * L
            continue
        I, J = np.nonzero(np.asarray(block_mask))
        r0 = I.astype(np.int64) * mask_block
        r1 = np.minimum(r0 + mask_block, N)
        c0 = J.astype(np.int64) * mask_block
        c1 = np.minimum(c0 + mask_block, L)
        keep = c1 > c0
        r0, r1, c0, c1 = r0[keep], r1[keep], c0[keep], c1[keep]
        if not causal:
            total += int(((r1 - r0) * (c1 - c0)).sum())
        else:
            for a, b_, c, e in zip(r0, r1, c0, c1):
                i = np.arange(a, b_)
                total += int(np.clip(np.minimum(i + 1 + off, e) - c, 0, None).sum())
    return total * H


def kernel_bytes(B, H, N, d, esize, seqlens, Nk=None):
    """Compulsory HBM bytes per call of each pass: every tensor the pass must
    read or write once (keys and values only up to each sequence's key
    length), plus the fp32 row statistics: L, and for the backward pass D
    (written by its first kernel, read by its second).  N queries, Nk keys
    (default N)."""
    Nk = N if Nk is None else Nk
    t = B * H * N * d * esize
    tk = B * H * Nk * d * esize
    kv_valid = H * d * esize * (B * Nk if seqlens is None
                                else int(np.minimum(seqlens, Nk).sum()))
    rowstat = B * H * N * 4
    return {
        "fa_fwd": 2 * t + 2 * kv_valid + rowstat,    # Q, O; K, V; L
        # Q, O, dO, dQ; dK, dV; K, V; L; D written and read
        "fa_bwd": 4 * t + 2 * tk + 2 * kv_valid + 3 * rowstat,
    }


def kernel_flops(d, pairs):
    """Algorithmic FLOPs per call: the forward pass is two products over the
    visible pairs (S, O; 2*d each), the backward pass five (S recomputed, dV,
    dP, dQ, dK).  The backward kernel's second recomputation of S and dP (in
    its dQ workgroups) duplicates work and is not credited."""
    return {"fa_fwd": 4.0 * d * pairs, "fa_bwd": 10.0 * d * pairs}


# ------------------------------------------------------------------- timing

# The two C calls of a step and the kernels each launches, in order: fa_bwd
# writes D = rowsum(dO * O) with dsum_kernel, then runs bwd_kernel.
PASSES = ("fa_fwd", "fa_bwd")
PASS_KERNELS = {"fa_fwd": ("fwd_bf16_kernel",), "fa_bwd": ("dsum_kernel", "bwd_kernel")}
# the fp32 path's kernels per C call
PASS_KERNELS_F32 = {"fa_fwd": ("fwd_f32_kernel",), "fa_bwd": ("dq_f32_kernel", "dkdv_f32_kernel")}


def pass_kernels(dtype: str) -> dict:
    return PASS_KERNELS if dtype == "bf16" else PASS_KERNELS_F32


DROPOUT_SEED = 2024  # Philox key of the --dropout runs (offset 0)


def measure_key(workload: str, dropout_p: float) -> str:
    """Name of the profiles/ records of a run: the workload, plus the drop
    probability when dropout is on (a different kernel variant)."""
    return workload if dropout_p <= 0 else f"{workload}_dropout{dropout_p:g}"


def run_gpu(w: wl.Workload, inp: dict, steps: int, warmup: int, prewarm_s: float = 1.0,
            dropout_p: float = 0.0, cold_reps: int = 0, event_reps: int = 50,
            restricted_rerun: bool = True, graph: bool = False):
    """Times `steps` steps after `warmup` untimed ones.  One step is fa_fwd
    then fa_bwd (fa_fwd alone for a forward-only workload), each a single
    kernel launch on the current stream; the wall clock around the timed
    steps (synchronised on both sides) gives the step time.  With `graph`
    the step's calls are recorded once into a HIP graph (captured on a side
    stream) and every prewarm, warmup and timed step is one replay of it:
    the host then submits one graph instead of each call's launches.

    Before the warmup steps the step runs untimed for `prewarm_s` seconds of
    wall time: an idle MI355X takes a few milliseconds of sustained load to
    raise its clocks, and a short warmup would otherwise time the ramp.

    Each kernel's device time comes from `event_reps` further steps, run
    after the timed ones and outside their wall clock, with a HIP event
    recorded on the launch stream before the step's first launch and after
    each launch (event packets cost the stream a few microseconds, so they
    stay out of the timed steps).

    Then `cold_reps` launches of each kernel are timed one by one, each right
    after a FLUSH_BYTES write on the same stream (the kernel then starts with
    nothing of its inputs in L2 or the Infinity Cache); their medians are
    returned as cold_ms."""
    import torch
    import exact_io_aware_64_amd as fa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    to = lambda x: torch.from_numpy(x).to(tdt).to(dev)  # noqa: E731
    q, k, v, do = (to(inp[n]) for n in ("q", "k", "v", "do"))
    sl = None if inp["seqlens"] is None else torch.from_numpy(inp["seqlens"]).to(dev)
    bm = None if inp["block_mask"] is None else torch.from_numpy(inp["block_mask"]).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    kw = dict(scale=w.scale, causal=w.causal, seqlens_k=sl, block_mask=bm, mask_block=128,
              dropout_p=dropout_p, seed=DROPOUT_SEED, offset=0)
    stream = torch.cuda.current_stream(dev)
    # argument marshalling done once, so the host keeps ahead of the GPU
    fwd = fa.prepare_fwd(q, k, v, o, lse, **kw)
    bwd = fa.prepare_bwd(q, k, v, o, do, lse, dq, dk, dv, **kw) if w.backward else None
    kernels = PASSES if w.backward else PASSES[:1]

    # ev: [start, after launch 0, after launch 1, ...] of a sampled step
    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fwd()
        if ev is not None:
            ev[1].record(stream)
        if bwd is not None:
            bwd()
            if ev is not None:
                ev[2].record(stream)

    timed_step = step
    if graph:
        side = torch.cuda.Stream(device=dev)
        fwd_s = fa.prepare_fwd(q, k, v, o, lse, stream=side.cuda_stream, **kw)
        bwd_s = (fa.prepare_bwd(q, k, v, o, do, lse, dq, dk, dv, stream=side.cuda_stream, **kw)
                 if w.backward else None)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):  # first calls outside the capture
            fwd_s()
            if bwd_s is not None:
                bwd_s()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            fwd_s()
            if bwd_s is not None:
                bwd_s()
        timed_step = g.replay

    torch.cuda.synchronize()
    t_end = time.perf_counter() + prewarm_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            timed_step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        timed_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        timed_step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)]
           for _ in range(max(1, event_reps))]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    durs = launch_durations(evs, kernels)
    kernel_ms = {name: float(np.mean(d)) for name, d in durs.items()}
    median_ms = {name: float(np.median(d)) for name, d in durs.items()}
    cold_ms = None
    if cold_reps > 0:
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        launches = [fwd] + ([bwd] if bwd is not None else [])
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(launches))]
               for _ in range(cold_reps)]
        for r, e in enumerate(cev):
            for i, f in enumerate(launches):
                flush.fill_(r & 0xFF)
                e[2 * i].record(stream)
                f()
                e[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        cold_ms = {name: float(np.median([e[2 * i].elapsed_time(e[2 * i + 1]) for e in cev]))
                   for i, name in enumerate(kernels)}
        del flush
    # the same outputs again (the last launches wrote them), and for sampled
    # workloads the backward pass rerun with dO kept on the sampled rows only
    # (its dK, dV are the oracle's restricted gradients)
    restricted = None
    if restricted_rerun and bwd is not None and inp.get("rows") is not None:
        rows = torch.from_numpy(inp["rows"]).to(dev)
        do_r = torch.zeros_like(do)
        idx = rows[..., None].expand(-1, -1, -1, do.shape[-1])
        do_r.scatter_(2, idx, do.gather(2, idx))
        dq_r, dk_r, dv_r = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        fa.prepare_bwd(q, k, v, o, do_r, lse, dq_r, dk_r, dv_r, **kw)()
        torch.cuda.synchronize()
        restricted = dict(dk=dk_r, dv=dv_r)
        del do_r, dq_r
    props = torch.cuda.get_device_properties(dev)
    outs = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, restricted=restricted)
    return wall_ms, kernel_ms, median_ms, cold_ms, props, outs


def launch_durations(samples, kernels) -> dict:
    """Per-kernel durations (ms) of the sampled steps: samples[i][0] was
    recorded right before the step's first launch and samples[i][j + 1] right
    after its launch j, so launch j ran between samples[i][j] and
    samples[i][j + 1]."""
    durs = {name: [] for name in kernels}
    for e in samples:
        for j, name in enumerate(kernels):
            durs[name].append(e[j].elapsed_time(e[j + 1]))
    return durs


def host_info() -> dict:
    """CPU model and the BLAS library NumPy runs on (for the CPU baseline)."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:  # pragma: no cover
        pass
    return dict(cpu=model, blas=blas)


def sampled_pairs(rows, N: int, causal: bool, seqlens, block_mask, mask_block: int = 128,
                  Nk=None) -> int:
    """Visible (query, key) pairs of the query rows ``rows`` (int ``[B, H, R]``),
    summed over batch and heads: N queries, Nk keys (default N), causal key j
    visible to query i iff j <= i + Nk - N."""
    Nk = N if Nk is None else Nk
    rows = np.asarray(rows, dtype=np.int64)
    B = rows.shape[0]
    total = 0
    for b in range(B):
        L = Nk if seqlens is None else int(min(max(int(seqlens[b]), 0), Nk))
        r = rows[b].reshape(-1)
        lim = np.full(r.shape, L, dtype=np.int64)
        if causal:
            lim = np.minimum(lim, r + 1 + Nk - N)
        lim = np.maximum(lim, 0)
        if block_mask is None:
            total += int(lim.sum())
            continue
        bm = np.asarray(block_mask).astype(bool)
        c0 = np.arange(bm.shape[1], dtype=np.int64) * mask_block
        over = np.clip(np.minimum(c0[None, :] + mask_block, lim[:, None]) - c0[None, :], 0, None)
        total += int((bm[r // mask_block] * over).sum())
    return total


def cpu_baseline(w: wl.Workload, inp: dict, outs: dict, flops_fb: float,
                 budget_s: float = 10.0, dropout_p: float = 0.0):
    """The fp64 oracle as it stands, on the host cores, on the same inputs.

    Sample: for workloads that name sampled query rows (the 16K and 64K
    ones), those rows of the first heads -- the oracle's forward and
    backward restricted to them (O, L, dQ of the rows; dK, dV of the problem
    with dO kept on the rows only) -- else whole (batch, head) slices; all
    heads when one pass fits the budget, repeated until about ``budget_s``
    seconds of CPU work.  The value is the visible-pair FLOPs of what was
    computed over the time taken; the full-problem time at that rate is an
    extrapolation unless the sample was the whole workload."""
    from oracle import attention_ref as ref
    from oracle import dropout_ref as dref
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    args = dict(causal=w.causal, seqlens=inp["seqlens"], block_mask=inp["block_mask"],
                mask_block=128)
    H = w.H
    rows = inp.get("rows")
    sampled = rows is not None
    sub = lambda x, hs: x[:, :hs]  # noqa: E731
    per_pair = 4.0 * w.d + (10.0 * w.d if w.backward else 0.0)

    def one_pass(hs):
        q, k, v, do = (sub(inp[n], hs) for n in ("q", "k", "v", "do"))
        rkw = dict(args, rows=sub(rows, hs)) if sampled else args
        if dropout_p > 0:  # mask index b * H + h with the workload's H
            dkw = dict(rkw, n_heads=H)
            O, L = dref.forward(q, k, v, w.scale, dropout_p, DROPOUT_SEED, 0, **dkw)
            G = dref.backward(q, k, v, do, w.scale, dropout_p, DROPOUT_SEED, 0, **dkw) \
                if w.backward else ()
            return O, L, G
        O, L = ref.forward(q, k, v, w.scale, **rkw)
        G = ref.backward(q, k, v, do, w.scale, **rkw) if w.backward else ()
        return O, L, G

    def flops_of(hs):
        if not sampled:
            return flops_fb * hs / H
        return per_pair * sampled_pairs(sub(rows, hs), w.N, w.causal, inp["seqlens"],
                                        inp["block_mask"], 128, Nk=w.n_keys)

    t0 = time.perf_counter()
    one_pass(1)
    per_head = time.perf_counter() - t0
    hs = int(max(1, min(H, budget_s / max(per_head, 1e-6))))
    passes = 0
    t0 = time.perf_counter()
    while True:
        O, L, G = one_pass(hs)
        passes += 1
        secs = time.perf_counter() - t0
        if secs >= budget_s or passes >= 50:
            break
    tflops = flops_of(hs) * passes / secs / 1e12
    # the same sample doubles as a parity spot check of the GPU outputs
    npf = lambda t: t[:, :hs].float().cpu().numpy().astype(np.float64)  # noqa: E731

    def at_rows(t):
        x = npf(t)
        if not sampled:
            return x
        r = sub(rows, hs)
        if x.ndim == 3:
            return np.take_along_axis(x, r, axis=2)
        return np.take_along_axis(x, r[..., None], axis=2)

    lg = at_rows(outs["lse"])
    fin = np.isfinite(L)
    parity = dict(O_maxabs=float(np.abs(at_rows(outs["o"]) - O).max()),
                  L_maxabs=float(np.abs(lg[fin] - L[fin]).max()) if fin.any() else 0.0)
    if G:
        gpu = dict(dQ=at_rows(outs["dq"]))
        if sampled:
            res = outs.get("restricted")
            if res is not None:
                gpu.update(dK=npf(res["dk"]), dV=npf(res["dv"]))
        else:
            gpu.update(dK=npf(outs["dk"]), dV=npf(outs["dv"]))
        for name, g in zip(("dQ", "dK", "dV"), G):
            if name in gpu:
                parity[f"{name}_relfro"] = float(np.linalg.norm(gpu[name] - g)
                                                 / np.linalg.norm(g))
        if sampled:
            parity["sample"] = (f"{rows.shape[-1]} query rows per head on {hs} heads; dK, dV "
                                f"from the backward rerun with dO kept on those rows")
    full_s = flops_fb / (tflops * 1e12)
    whole = (not sampled) and hs == H
    what = (f"{rows.shape[-1]} sampled query rows per head (dK, dV of dO restricted to them)"
            if sampled else "whole sequences")
    base = dict(value=tflops, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"fp64 NumPy oracle {'fwd+bwd' if w.backward else 'fwd'} on {hs} of "
                       f"{H} heads x batch {w.B}, {what}, {passes} pass(es) in {secs:.1f} s; "
                       f"value = visible-pair FLOPs of the sample / time",
                seconds=secs,
                full_problem_s=full_s,
                full_problem_s_kind="measured" if whole else "extrapolated from the sample",
                **host_info())
    return base, parity


def copy_calibration(mib: int, steps: int, warmup: int) -> int:
    """A plain device-to-device copy of known size, used to scale HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) read under rocprofv3."""
    import torch
    n = mib << 20
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    y = torch.empty_like(x)
    for _ in range(warmup):
        y.copy_(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n,
                      "ms": dt * 1e3, "GBps_read_plus_write": 2 * n / dt / 1e9}), flush=True)
    return 0


# ------------------------------------------------------------ IO sweep

SWEEP_N = (1024, 2048, 4096, 8192, 16384, 32768)
SWEEP_BQ = (64, 128, 256)
SWEEP_B, SWEEP_H, SWEEP_D = 1, 16, 64
SWEEP_SEED = 6
SWEEP_REPS = 3


def sweep_model(N: int, block_q: int, H: int = SWEEP_H, d: int = SWEEP_D) -> dict:
    """Bytes of one dense (non-causal) bf16 forward of B = 1: the compulsory
    traffic (Q, K, V read once, O written once, L) and the K/V bytes the
    kernel streams through LDS, once per query tile: (N / block_q) * 2 N d * 2
    per head, the N^2 d / Br term of the pages' IO count."""
    t = N * d * 2
    nqt = -(-N // block_q)
    return dict(compulsory=H * (4 * t + 4 * N), compulsory_read=H * 3 * t,
                kv_streamed=H * nqt * 2 * t, q_read=H * t)


def io_sweep_run(ns, bqs, reps: int) -> int:
    """Dense bf16 forward (B=1, H=16, d=64) for every N and query-tile height:
    one untimed and `reps` event-timed fa_fwd_tiled launches each, in a fixed
    order, one JSON line per configuration.  Under rocprofv3 --pmc the
    dispatches are told apart by workgroup size (block_q / 32 waves per group
    of waves, times the key-range groups) and grid size (N / block_q * H
    workgroups), both recorded in the line."""
    import torch
    import exact_io_aware_64_amd as fa
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(SWEEP_SEED)
    nmax = max(ns)
    full = [torch.from_numpy(x).to(torch.bfloat16).to(dev)
            for x in wl.draw_tensors(rng, SWEEP_B, SWEEP_H, nmax, SWEEP_D, "bf16", count=3)]
    stream = torch.cuda.current_stream(dev)
    for N in ns:
        q, k, v = (x[:, :, :N] for x in full)
        o = torch.empty((SWEEP_B, SWEEP_H, N, SWEEP_D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((SWEEP_B, SWEEP_H, N), dtype=torch.float32, device=dev)
        for bq in bqs:
            call = fa.prepare_fwd_tiled(q, k, v, o, lse, scale=1 / 8, block_q=bq)
            call()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(reps)]
            for a, b in evs:
                a.record(stream)
                call()
                b.record(stream)
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
            flops = 4.0 * SWEEP_D * N * N * SWEEP_H * SWEEP_B
            groups = fa.fa_fwd_key_groups(fa.FA_BF16, SWEEP_B, SWEEP_H, N, N, SWEEP_D, bq)
            print(json.dumps(dict(mode="io-sweep", N=N, block_q=bq, ms=ms,
                                  tflops=flops / (ms * 1e-3) / 1e12,
                                  workgroups=-(-N // bq) * SWEEP_H * SWEEP_B,
                                  threads=2 * bq * groups, key_groups=groups,
                                  **sweep_model(N, bq))), flush=True)
    return 0


def _per_dispatch(path: str, counters):
    """{dispatch id: dict(kernel, grid, wg, counter values summed over
    dimensions)} from a rocprofv3 counter_collection.csv."""
    out = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] not in counters:
                continue
            d = out.setdefault(int(row["Dispatch_Id"]), dict(
                kernel=_short_kernel_name(row["Kernel_Name"]), name=row["Kernel_Name"],
                grid=int(row["Grid_Size"]), wg=int(row["Workgroup_Size"])))
            d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return out


def _sweep_config(d, shapes):
    """(N, block_q) of a sweep dispatch from its launch shape: `shapes` maps
    (workgroups, threads per workgroup) of each configuration the sweep log
    records to (N, block_q)."""
    return shapes[(d["grid"] // d["wg"], d["wg"])]


def io_sweep_summary(fetch_csv, write_csv, l2_csv, cfetch_csv, cwrite_csv, cl2_csv, log,
                     command, copy_bytes) -> str:
    """profiles/io_sweep.md: measured bytes per launch of every sweep
    configuration (means over its dispatches), against the model."""
    def copy_max(path, counter):
        vals = [v[counter] for v in _per_dispatch(path, (counter,)).values()]
        return max(vals)
    f_fetch = copy_bytes / (copy_max(cfetch_csv, "FETCH_SIZE") * 1024.0)
    f_write = copy_bytes / (copy_max(cwrite_csv, "WRITE_SIZE") * 1024.0)
    f_sect = copy_bytes / copy_max(cl2_csv, "TCC_READ_SECTORS_sum")
    timing, shapes = {}, {}
    with open(log) as fh:
        for line in fh:
            if line.startswith("{") and '"io-sweep"' in line:
                r = json.loads(line)
                timing[(r["N"], r["block_q"])] = r
                shapes[(r["workgroups"], r["threads"])] = (r["N"], r["block_q"])
    meas = {}
    for path, counters in ((fetch_csv, ("FETCH_SIZE",)), (write_csv, ("WRITE_SIZE",)),
                           (l2_csv, ("TCC_READ_SECTORS_sum", "TCC_HIT_sum", "TCC_MISS_sum"))):
        for d in _per_dispatch(path, counters).values():
            if d["kernel"] != "fwd_bf16_kernel":
                continue
            acc = meas.setdefault(_sweep_config(d, shapes), {})
            for c in counters:
                acc.setdefault(c, []).append(d.get(c, 0.0))
    rows = []
    for (N, bq) in sorted(meas):
        m = {c: float(np.mean(v)) for c, v in meas[(N, bq)].items()}
        mod = sweep_model(N, bq)
        fetch = m["FETCH_SIZE"] * 1024.0 * f_fetch
        write = m["WRITE_SIZE"] * 1024.0 * f_write
        l2 = m["TCC_READ_SECTORS_sum"] * f_sect
        hit = m["TCC_HIT_sum"] / max(1.0, m["TCC_HIT_sum"] + m["TCC_MISS_sum"])
        t = timing.get((N, bq), {})
        rows.append((N, bq, t.get("key_groups", 1), mod["compulsory"] / 1e6,
                     (mod["q_read"] + mod["kv_streamed"]) / 1e6,
                     l2 / 1e6, fetch / 1e6, write / 1e6, fetch / mod["compulsory_read"], hit,
                     t.get("ms", float("nan")) * 1e3, t.get("tflops", float("nan"))))
    out = ["# IO sweep: dense bf16 forward, B=1 H=16 d=64, query tile height x N", "",
           "Command (repository root, MI355X, `TMPDIR=/tmp`):", "", "```", command, "```", "",
           "Model (per launch): *compulsory* = Q, K, V read once + O written once + L; "
           "*streamed* = Q + K/V read once per query tile, (N / Br) * 2 N d * 2 bytes per "
           "head -- the N^2 d / Br term of the pages' IO count.  Measured: *L2 read* = "
           "TCC_READ_SECTORS (bytes the CUs read from L2), *fetch* = FETCH_SIZE (bytes L2 "
           "read from memory, Infinity Cache hits included), *write* = WRITE_SIZE; each "
           f"scaled by the same counter over a {copy_bytes >> 20} MiB device copy "
           f"(factors: sectors x {f_sect:.2f} B, fetch x {f_fetch:.3f}, write x {f_write:.3f}). "
           "Time: median of event-timed launches in the same run.  Groups: key-range groups "
           "per query tile (3 when the grid has no more query tiles than the GPU has CUs; "
           "each still streams its share of K/V once per query tile, so the model holds).",
           "",
           "| N | Br | groups | compulsory MB | streamed MB (model) | L2 read MB | fetch MB "
           "| write MB | fetch / compulsory read | L2 hit rate | us | TFLOP/s |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| %d | %d | %d | %.1f | %.1f | %.1f | %.1f | %.1f | %.2f | %.3f | %.1f | %.0f |"
                   % r)
    return "\n".join(out) + "\n"


# ------------------------------------------------------- HBM bytes vs N

HBM_N = (1024, 2048, 4096, 8192, 16384, 32768, 65536)
HBM_B, HBM_H, HBM_D = 1, 8, 64
HBM_KINDS = ("causal", "blocksparse")
HBM_SEED = 11
HBM_REPS = 3
# Requests that leave L2 for memory, in 32-byte units (gfx950 TCC counters):
# reads and writes whose address is in the GPU's own HBM.
DRAM_COUNTERS = ("TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")


def _template_args(name: str):
    """Template arguments of a demangled kernel name, as strings."""
    if "<" not in name:
        return []
    inner = name[name.index("<") + 1:name.index(">")]
    return [a.strip() for a in inner.split(",")]


def _has_block_mask(kernel: str, name: str) -> bool:
    """Whether a dispatch ran the block-mask instantiation: the fifth template
    argument of fwd_bf16_kernel<W, G, D, SEQLEN, BMASK, DROP>, the fourth of
    bwd_kernel<D, CAUSAL, SEQLEN, BMASK, DROP>."""
    args = _template_args(name)
    pos = 4 if kernel == "fwd_bf16_kernel" else 3
    return len(args) > pos and args[pos] == "true"


def hbm_sweep_run(ns, kinds, reps: int) -> int:
    """fa_fwd and fa_bwd on B=1, H=8, d=64 for every N and mask kind (causal;
    block-sparse: 128 x 128 tiles, diagonal plus each off-diagonal tile with
    p = 1/16, non-causal): one untimed and `reps` event-timed launches of
    each, in a fixed order, one JSON line per configuration.  Under rocprofv3
    --pmc a dispatch is told apart by kernel, block-mask instantiation and
    workgroup count, all recorded in the line."""
    import torch
    import exact_io_aware_64_amd as fa
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rng = np.random.default_rng(HBM_SEED)
    nmax = max(ns)
    full = wl.draw_tensors(rng, HBM_B, HBM_H, nmax, HBM_D, "bf16", count=4)
    for N in ns:
        q, k, v, do = (torch.from_numpy(np.ascontiguousarray(x[:, :, :N])).to(torch.bfloat16)
                       .to(dev) for x in full)
        for kind in kinds:
            causal = kind == "causal"
            bm_np = None if causal else wl.draw_block_mask(
                np.random.default_rng(HBM_SEED + N), N, 1 / 16)
            bm = None if bm_np is None else torch.from_numpy(bm_np).to(dev)
            o = torch.empty_like(q)
            lse = torch.empty((HBM_B, HBM_H, N), dtype=torch.float32, device=dev)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            kw = dict(scale=1 / 8, causal=causal, block_mask=bm)
            fwd = fa.prepare_fwd(q, k, v, o, lse, **kw)
            bwd = fa.prepare_bwd(q, k, v, o, do, lse, dq, dk, dv, **kw)
            fwd()
            bwd()
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
            for e in evs:
                e[0].record(stream)
                fwd()
                e[1].record(stream)
                bwd()
                e[2].record(stream)
            torch.cuda.synchronize()
            fms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
            bms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
            pairs = visible_pairs(N, HBM_H, causal, None, bm_np, 128, HBM_B)
            kb = kernel_bytes(HBM_B, HBM_H, N, HBM_D, 2, None)
            nqt = -(-N // 128)
            groups = fa.fa_fwd_key_groups(fa.FA_BF16, HBM_B, HBM_H, N, N, HBM_D, 128)
            print(json.dumps(dict(
                mode="hbm-sweep", N=N, kind=kind, pairs=pairs, fwd_ms=fms, bwd_ms=bms,
                fwd_tflops=4.0 * HBM_D * pairs / (fms * 1e-3) / 1e12,
                bwd_tflops=10.0 * HBM_D * pairs / (bms * 1e-3) / 1e12,
                fwd_workgroups=nqt * HBM_B * HBM_H, fwd_threads=256 * groups,
                bwd_workgroups=2 * nqt * HBM_B * HBM_H,
                compulsory_fwd=kb["fa_fwd"], compulsory_bwd=kb["fa_bwd"])),
                flush=True)
            del o, lse, dq, dk, dv, fwd, bwd
        del q, k, v, do
    return 0


def hbm_sweep_summary(fetch_csv, write_csv, dram_csv, cfetch_csv, cwrite_csv, cdram_csv, log,
                      command, copy_bytes, mall_csv=None, mall_log=None) -> str:
    """profiles/hbm_vs_n.md: bytes per launch of fa_fwd and fa_bwd across N and
    mask kind (means over each configuration's dispatches), four counters,
    each scaled by what it reads for a plain device copy of known size."""
    def copy_max(path, counter):
        return max(v[counter] for v in _per_dispatch(path, (counter,)).values())
    f_fetch = copy_bytes / (copy_max(cfetch_csv, "FETCH_SIZE") * 1024.0)
    f_write = copy_bytes / (copy_max(cwrite_csv, "WRITE_SIZE") * 1024.0)
    f_drd = copy_bytes / copy_max(cdram_csv, DRAM_COUNTERS[0])
    f_dwr = copy_bytes / copy_max(cdram_csv, DRAM_COUNTERS[1])
    cfg = {}
    with open(log) as fh:
        for line in fh:
            if line.startswith("{") and '"hbm-sweep"' in line:
                r = json.loads(line)
                bmask = r["kind"] == "blocksparse"
                cfg[("fwd_bf16_kernel", bmask, r["fwd_workgroups"])] = r
                cfg[("bwd_kernel", bmask, r["bwd_workgroups"])] = r
    meas = {}
    for path, counters in ((fetch_csv, ("FETCH_SIZE",)), (write_csv, ("WRITE_SIZE",)),
                           (dram_csv, DRAM_COUNTERS)):
        disp = _per_dispatch(path, counters)
        # a pass's counts: its kernels' dispatches summed; dsum_kernel is
        # charged to the bwd_kernel dispatch that follows it
        pending = {c: 0.0 for c in counters}
        for i in sorted(disp):
            d = disp[i]
            if d["kernel"] == "dsum_kernel":
                for c in counters:
                    pending[c] += d.get(c, 0.0)
                continue
            if d["kernel"] not in ("fwd_bf16_kernel", "bwd_kernel"):
                continue
            key = (d["kernel"], _has_block_mask(d["kernel"], d["name"]), d["grid"] // d["wg"])
            extra = pending if d["kernel"] == "bwd_kernel" else {c: 0.0 for c in counters}
            if d["kernel"] == "bwd_kernel":
                pending = {c: 0.0 for c in counters}
            if key not in cfg:
                continue
            r = cfg[key]
            acc = meas.setdefault((r["N"], r["kind"], d["kernel"]), {})
            for c in counters:
                acc.setdefault(c, []).append(d.get(c, 0.0) + extra[c])
    rows = []
    for (N, kind, kern) in sorted(meas, key=lambda x: (x[1], x[2] != "fwd_bf16_kernel", x[0])):
        m = {c: float(np.mean(v)) for c, v in meas[(N, kind, kern)].items()}
        fwd = kern == "fwd_bf16_kernel"
        r = next(v for v in cfg.values() if v["N"] == N and v["kind"] == kind)
        comp = r["compulsory_fwd" if fwd else "compulsory_bwd"]
        fetch = m.get("FETCH_SIZE", float("nan")) * 1024.0 * f_fetch
        write = m.get("WRITE_SIZE", float("nan")) * 1024.0 * f_write
        drd = m.get(DRAM_COUNTERS[0], float("nan")) * f_drd
        dwr = m.get(DRAM_COUNTERS[1], float("nan")) * f_dwr
        us = 1e3 * r["fwd_ms" if fwd else "bwd_ms"]
        rows.append((kind, "fwd" if fwd else "bwd", N, us,
                     r["fwd_tflops" if fwd else "bwd_tflops"], comp / 1e6, fetch / 1e6,
                     write / 1e6, drd / 1e6, dwr / 1e6, (fetch + write) / comp,
                     (drd + dwr) / comp, (drd + dwr) / N / 1e3))
    out = ["# HBM bytes vs N: fa_fwd and fa_bwd, B=1 H=8 d=64, causal and block-sparse", "",
           "Command (repository root, MI355X, `TMPDIR=/tmp`):", "", "```", command, "```", "",
           "Per call, mean over the configuration's calls (one untimed and three timed "
           "calls each; the backward call's two kernels, dsum_kernel and bwd_kernel, "
           "summed).  *compulsory* = every tensor the pass must read or write once "
           "(forward: Q, K, V, O and L; backward: Q, K, V, O, dO, L, dQ, dK, dV, and D "
           "written and read once).  Measured: "
           "*fetch* = FETCH_SIZE and *write* = WRITE_SIZE (bytes leaving L2 toward memory); "
           "*DRAM rd* = TCC_EA0_RDREQ_DRAM_32B and *DRAM wr* = TCC_EA0_WRREQ_WRITE_DRAM_32B "
           "(requests leaving L2 whose address lies in the GPU's own HBM, 32-byte units).  "
           "Each is scaled by the same counter over a "
           f"{copy_bytes >> 20} MiB device copy (factors: fetch x {f_fetch:.3f}, write x "
           f"{f_write:.3f}, DRAM rd x {f_drd:.2f} B, DRAM wr x {f_dwr:.2f} B).  Block-sparse: "
           "128 x 128 tile mask, diagonal plus each off-diagonal tile with p = 1/16, "
           "non-causal.  Time: median of the timed launches (events) in the same run.", "",
           "| mask | pass | N | us | TFLOP/s | compulsory MB | fetch MB | write MB | DRAM rd MB "
           "| DRAM wr MB | (fetch+write) / compulsory | DRAM / compulsory | DRAM KB per row |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| %s | %s | %d | %.1f | %.0f | %.1f | %.1f | %.1f | %.1f | %.1f | %.2f | "
                   "%.2f | %.1f |" % r)
    if mall_csv and mall_log:
        sizes = []
        with open(mall_log) as fh:
            for line in fh:
                if line.startswith("{") and '"copy"' in line:
                    sizes.append(json.loads(line))
        if sizes:
            c = sizes[-1]
            # the copies, not the fill that initialises the source
            big = [d for d in _per_dispatch(mall_csv, DRAM_COUNTERS).values()
                   if "fill" not in d["name"].lower()]
            rd = float(np.median([d[DRAM_COUNTERS[0]] for d in big])) * f_drd
            wr = float(np.median([d[DRAM_COUNTERS[1]] for d in big])) * f_dwr
            out += ["", "Infinity Cache probe: a plain copy of "
                    f"{c['bytes_read'] >> 20} MiB (larger than the 8 x 4 MB of L2, smaller than "
                    f"the 256 MB Infinity Cache), repeated: {c['ms'] * 1e3:.1f} us per copy, "
                    f"{c['GBps_read_plus_write']:.0f} GB/s read + write; DRAM rd "
                    f"{rd / 1e6:.1f} MB and DRAM wr {wr / 1e6:.1f} MB per copy (median over "
                    f"{len(big)} dispatches)."]
    return "\n".join(out) + "\n"


# ------------------------------------------------------------ HBM traffic

KERNEL_SOURCES = {
    "fwd_bf16_kernel": ("fa_fwd_bf16.hip",),
    "dsum_kernel": ("fa_bwd_bf16.h", "fa_bwd_bf16.hip", "fa_bwd_bf16_d128.hip"),
    "bwd_kernel": ("fa_bwd_bf16.h", "fa_bwd_bf16.hip", "fa_bwd_bf16_d128.hip"),
    "fwd_f32_kernel": ("fa_f32_tile.h", "fa_fwd_f32.hip"),
    "dq_f32_kernel": ("fa_f32_tile.h", "fa_bwd_f32.hip"),
    "dkdv_f32_kernel": ("fa_f32_tile.h", "fa_bwd_f32.hip"),
}
COMMON_SOURCES = ("fa_device.h", "fa_internal.h")


def kernel_source_hash(kernel: str) -> str:
    """sha256 over the sources a kernel is compiled from and the compiler
    flags of its translation units."""
    from exact_io_aware_64_amd import build as B
    pkg = os.path.join(ROOT, "exact_io_aware_64_amd")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + COMMON_SOURCES:
        with open(os.path.join(pkg, "csrc", f), "rb") as fh:
            h.update(fh.read())
        if f.endswith(".hip"):
            h.update(" ".join(B.source_flags(f)).encode())
    return h.hexdigest()


def _short_kernel_name(name: str) -> str:
    name = name.replace("void ", "").replace("fa::(anonymous namespace)::", "")
    return name.split("(")[0].split("<")[0].strip()


def read_counter_csv(path: str, counter: str):
    """Mean value per dispatch of `counter` for each kernel of a rocprofv3
    counter_collection.csv, keyed by the kernel's short name."""
    per = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            k = _short_kernel_name(row["Kernel_Name"])
            per.setdefault(k, {}).setdefault(row["Dispatch_Id"], 0.0)
            per[k][row["Dispatch_Id"]] += float(row["Counter_Value"])
    return {k: (float(np.mean(list(v.values()))), len(v)) for k, v in per.items()}


def pmc_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, workload, copy_bytes,
                command):
    """Builds the traffic record: per-kernel FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch) scaled by what the same counters read for a copy kernel that
    moves copy_bytes in and copy_bytes out."""
    f = read_counter_csv(fetch_csv, "FETCH_SIZE")
    wr = read_counter_csv(write_csv, "WRITE_SIZE")
    cf = read_counter_csv(copy_fetch_csv, "FETCH_SIZE")
    cw = read_counter_csv(copy_write_csv, "WRITE_SIZE")
    # the copy is the dispatch with the largest counter value
    cf_kib = max(v for v, _ in cf.values())
    cw_kib = max(v for v, _ in cw.values())
    f_fetch = copy_bytes / (cf_kib * 1024.0)
    f_write = copy_bytes / (cw_kib * 1024.0)
    kernels = {}
    for k in KERNEL_SOURCES:
        if k not in f or k not in wr:
            continue
        fk, nf = f[k]
        wk, nw = wr[k]
        kernels[k] = dict(fetch_kib=fk, write_kib=wk, dispatches=[nf, nw],
                          fetch_bytes=fk * 1024.0 * f_fetch, write_bytes=wk * 1024.0 * f_write,
                          bytes_per_launch=fk * 1024.0 * f_fetch + wk * 1024.0 * f_write,
                          source_sha256=kernel_source_hash(k))
    return dict(workload=workload, command=command,
                copy_calibration=dict(bytes=copy_bytes, fetch_kib=cf_kib, write_kib=cw_kib,
                                      fetch_factor=f_fetch, write_factor=f_write),
                kernels=kernels)


def pipe_metrics(c: dict, n_cu: int = 256, simd_per_cu: int = 4, n_xcd: int = 8) -> dict:
    """Busy fractions of one dispatch from its counters, each summed over the
    GPU's block instances (as rocprofv3 reports them), with rocprofv3's own
    gfx950 formulas.  GRBM_GUI_ACTIVE counts the dispatch's active cycles once
    per XCD, so the dispatch lasted gui = GRBM_GUI_ACTIVE / n_xcd cycles.
    MFMA busy = MFMA busy cycles / (gui x SIMDs); VALU busy = VALU-active
    quad-cycles / (gui x CUs), the share of SIMD cycles executing a vector
    instruction; CU busy = CU-busy cycles / (gui x CUs); LDS bank-conflict
    share = conflict cycles / LDS-active cycles."""
    gui = c["GRBM_GUI_ACTIVE"] / n_xcd
    return dict(
        mfma_busy=c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * n_cu * simd_per_cu),
        valu_busy=c["SQ_ACTIVE_INST_VALU"] / (gui * n_cu),
        lds_conflict=c["SQ_LDS_BANK_CONFLICT"] / max(1.0, c["SQ_LDS_IDX_ACTIVE"]),
        trans_per_mfma=c["SQ_INSTS_VALU_TRANS_F32"] / max(1.0, c["SQ_INSTS_MFMA"]),
        cu_busy=c["SQ_BUSY_CU_CYCLES"] / (gui * n_cu),
        gui_cycles=gui)


def pipe_summary(counter_csv: str, workload: str, command: str) -> str:
    """Markdown summary of a rocprofv3 --pmc run over PIPE_COUNTERS: per
    kernel, the counters averaged over its dispatches (each summed over the
    GPU's instances) and the busy fractions derived from them."""
    per = {}
    with open(counter_csv) as fh:
        for row in csv.DictReader(fh):
            k = _short_kernel_name(row["Kernel_Name"])
            if k not in KERNEL_SOURCES:
                continue
            d = per.setdefault(k, {}).setdefault(row["Dispatch_Id"], {})
            d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
            d["_ns"] = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
    out = [f"# Pipe counters: {workload}", "",
           "Command (repository root, MI355X, `TMPDIR=/tmp`):", "", "```", command, "```", "",
           "Per dispatch, averaged over the dispatches of the run (rocprofv3's gfx950 "
           "formulas; counters come summed over block instances, GRBM_GUI_ACTIVE once per "
           "XCD). µs: the dispatch's duration under the profiler; cycles: its active cycles; "
           "clock: the two divided. MFMA busy: share of SIMD cycles with the matrix core "
           "busy; VALU busy: share of SIMD cycles executing a vector instruction (MfmaUtil "
           "and VALUBusy); CU busy: share of CU cycles with waves resident; LDS conflict: "
           "bank-conflict cycles per LDS-active cycle; trans/MFMA: fp32 transcendental "
           "(exp2) instructions per MFMA instruction. A clock above the chip's 2.4 GHz "
           "(dispatches of a few µs, whose GRBM_GUI_ACTIVE window overlaps their "
           "neighbours) and trans/MFMA of a kernel without MFMAs are shown as —.", "",
           "| kernel | dispatches | µs | cycles | clock GHz | MFMA busy | VALU busy | CU busy | "
           "LDS conflict | trans/MFMA |", "|---|---|---|---|---|---|---|---|---|---|"]
    for k, disp in sorted(per.items()):
        full = [d for d in disp.values() if all(n in d for n in PIPE_COUNTERS)]
        if not full:
            continue
        mean = {n: float(np.mean([d[n] for d in full])) for n in PIPE_COUNTERS}
        ns = float(np.mean([d["_ns"] for d in full]))
        m = pipe_metrics(mean)
        clock = m["gui_cycles"] / ns
        clock_s = f"{clock:.2f}" if clock <= 2.45 else "—"
        tpm = f"{m['trans_per_mfma']:.2f}" if mean["SQ_INSTS_MFMA"] > 0 else "—"
        out.append(f"| {k} | {len(full)} | {ns / 1e3:.1f} | {m['gui_cycles']:.0f} | "
                   f"{clock_s} | {100 * m['mfma_busy']:.1f} % | "
                   f"{100 * m['valu_busy']:.1f} % | {100 * m['cu_busy']:.1f} % | "
                   f"{100 * m['lds_conflict']:.2f} % | {tpm} |")
    out += ["", "Raw means per dispatch:", ""]
    for k, disp in sorted(per.items()):
        full = [d for d in disp.values() if all(n in d for n in PIPE_COUNTERS)]
        if full:
            out.append(f"- {k}: " + ", ".join(
                f"{n} {np.mean([d[n] for d in full]):.4g}" for n in PIPE_COUNTERS))
    return "\n".join(out) + "\n"


def traffic_for(pass_name: str, workload: str, dtype: str = "bf16"):
    """Measured HBM bytes per call of a pass (the sum over its kernels) on
    `workload`, or None when no record exists or one of its kernels changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    total = 0.0
    for kernel in pass_kernels(dtype)[pass_name]:
        ent = rec.get("kernels", {}).get(kernel)
        if not ent or ent.get("source_sha256") != kernel_source_hash(kernel):
            return None
        total += float(ent["bytes_per_launch"])
    return total


def trace_summary(stats_csv: str, bench_log: str, workload: str, command: str) -> str:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of this
    script: per-kernel launch statistics and the JSON line the run printed."""
    rows = []
    with open(stats_csv) as fh:
        for row in csv.DictReader(fh):
            rows.append((_short_kernel_name(row["Name"]), int(row["Calls"]),
                         float(row["AverageNs"]) / 1e3, float(row["MinNs"]) / 1e3,
                         float(row["MaxNs"]) / 1e3, float(row["Percentage"])))
    line = None
    with open(bench_log) as fh:
        for l in fh:
            if l.startswith("{"):
                line = json.loads(l)
    out = [f"# Kernel trace: {workload}", "", "Command (repository root, MI355X, `TMPDIR=/tmp`):",
           "", "```", command, "```", "",
           "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for k, n, av, mn, mx, pc in rows:
        out.append(f"| {k} | {n} | {av:.2f} | {mn:.2f} | {mx:.2f} | {pc:.2f} |")
    avg = {k: av for k, n, av, mn, mx, pc in rows}
    per_call = [f"{p} = {' + '.join(ks)}: {sum(avg[k] for k in ks):.2f} us"
                for table in (PASS_KERNELS, PASS_KERNELS_F32)
                for p, ks in table.items() if all(k in avg for k in ks)]
    if per_call:
        out += ["", "Per C call (sum of its kernels' averages): " + "; ".join(per_call) + "."]
    if line:
        km = {k: round(v * 1e3, 2) for k, v in line["kernel_ms"].items()}
        out += ["", "Bench line of the same run (HIP events on the launch stream, us per call):",
                "", f"- kernels: {km}",
                (f"- fwd {line['fwd_tflops']:.1f} TFLOP/s, bwd {line['bwd_tflops']:.1f} "
                 f"TFLOP/s, fwd+bwd {line['value']:.1f} TFLOP/s "
                 f"({100 * line['fwdbwd_frac_peak']:.1f} % of {line['peak_tflops']})")
                if line.get("bwd_tflops") is not None else
                (f"- forward-only step: fwd {line['fwd_tflops']:.1f} TFLOP/s "
                 f"({100 * line['fwd_frac_peak']:.1f} % of {line['peak_tflops']})"),
                f"- roofline: {json.dumps(line['roofline'])}"]
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps (clock ramp)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=wl.WORKLOAD_ORDER)
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="drop probability on P (fa_fwd_dropout / fa_bwd_dropout); the FLOP "
                         "count is the same as without dropout")
    ap.add_argument("--cpu-baseline", default="on", choices=["on", "off"])
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of one HIP graph holding the step's calls")
    ap.add_argument("--event-reps", type=int, default=50,
                    help="steps after the timed ones whose launches are bracketed by HIP "
                         "events (per-kernel device time)")
    ap.add_argument("--cold-reps", type=int, default=50,
                    help="launches of each kernel timed after a 1 GiB cache-evicting write "
                         "(0: none)")
    ap.add_argument("--mode", default="attention",
                    choices=["attention", "copy", "io-sweep", "hbm-sweep"],
                    help="copy: time a plain 1 GiB device copy (counter calibration); "
                         "io-sweep: dense forward over N x query-tile height (fa_fwd_tiled); "
                         "hbm-sweep: fa_fwd + fa_bwd over N, causal and block-sparse")
    ap.add_argument("--sweep-n", default=",".join(str(n) for n in SWEEP_N))
    ap.add_argument("--io-summary", nargs=7, metavar=("FETCH_CSV", "WRITE_CSV", "L2_CSV",
                                                     "COPY_FETCH_CSV", "COPY_WRITE_CSV",
                                                     "COPY_L2_CSV", "SWEEP_LOG"),
                    help="write profiles/io_sweep.md from rocprofv3 runs of --mode io-sweep")
    ap.add_argument("--hbm-n", default=",".join(str(n) for n in HBM_N))
    ap.add_argument("--hbm-summary", nargs=7, metavar=("FETCH_CSV", "WRITE_CSV", "DRAM_CSV",
                                                      "COPY_FETCH_CSV", "COPY_WRITE_CSV",
                                                      "COPY_DRAM_CSV", "SWEEP_LOG"),
                    help="write profiles/hbm_vs_n.md from rocprofv3 runs of --mode hbm-sweep")
    ap.add_argument("--mall-probe", nargs=2, metavar=("DRAM_CSV", "COPY_LOG"),
                    help="with --hbm-summary: DRAM counters and log of a copy that fits the "
                         "Infinity Cache")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                     "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this script "
                         "(attention and --mode copy) into profiles/hbm_traffic_<workload>.json")
    ap.add_argument("--pmc-command", default="",
                    help="the rocprofv3 commands that produced the --pmc-summary inputs")
    ap.add_argument("--pipe-summary", metavar="COUNTER_CSV",
                    help="write profiles/pipe_counters_<workload>.md from a rocprofv3 "
                         "--pmc run of this script over PIPE_COUNTERS")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_STATS_CSV", "BENCH_LOG"),
                    help="write profiles/kernel_trace_<workload>.md from a rocprofv3 "
                         "--kernel-trace --stats run of this script")
    args = ap.parse_args(argv)
    key = measure_key(args.workload, args.dropout)
    if args.io_summary:
        md = io_sweep_summary(*args.io_summary, command=args.pmc_command,
                              copy_bytes=args.copy_mib << 20)
        with open(os.path.join(ROOT, "profiles", "io_sweep.md"), "w") as fh:
            fh.write(md)
        print(md)
        return 0
    if args.hbm_summary:
        mall = args.mall_probe or (None, None)
        md = hbm_sweep_summary(*args.hbm_summary, command=args.pmc_command,
                               copy_bytes=args.copy_mib << 20, mall_csv=mall[0],
                               mall_log=mall[1])
        with open(os.path.join(ROOT, "profiles", "hbm_vs_n.md"), "w") as fh:
            fh.write(md)
        print(md)
        return 0
    if args.trace_summary:
        md = trace_summary(*args.trace_summary, workload=key, command=args.pmc_command)
        with open(os.path.join(ROOT, "profiles", f"kernel_trace_{key}.md"), "w") as fh:
            fh.write(md)
        print(md)
        return 0
    if args.pipe_summary:
        md = pipe_summary(args.pipe_summary, workload=key, command=args.pmc_command)
        with open(os.path.join(ROOT, "profiles", f"pipe_counters_{key}.md"), "w") as fh:
            fh.write(md)
        print(md)
        return 0
    if args.pmc_summary:
        rec = pmc_summary(*args.pmc_summary, workload=key,
                          copy_bytes=args.copy_mib << 20, command=args.pmc_command)
        out = os.path.join(ROOT, "profiles", f"hbm_traffic_{key}.json")
        with open(out, "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps(rec["kernels"]), flush=True)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the attention path needs no collective "
              "(batch and heads shard across GPUs with no communication), so the figure "
              "is one MI355X's. Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.mode == "copy":
        return copy_calibration(args.copy_mib, args.steps, args.warmup)
    if args.mode == "io-sweep":
        return io_sweep_run([int(x) for x in args.sweep_n.split(",")], SWEEP_BQ, SWEEP_REPS)
    if args.mode == "hbm-sweep":
        return hbm_sweep_run([int(x) for x in args.hbm_n.split(",")], HBM_KINDS, HBM_REPS)

    w = wl.WORKLOADS[args.workload]
    inp = wl.make_inputs(w)
    pairs = visible_pairs(w.N, w.H, w.causal, inp["seqlens"], inp["block_mask"], 128, w.B,
                          Nk=w.n_keys)
    flops_f = 4.0 * w.d * pairs
    flops_b = 10.0 * w.d * pairs if w.backward else 0.0
    esize = 2 if w.dtype == "bf16" else 4

    wall_ms, kernel_ms, median_ms, cold_ms, props, outs = run_gpu(
        w, inp, args.steps, args.warmup, args.prewarm_s, args.dropout, args.cold_reps,
        args.event_reps, restricted_rerun=args.cpu_baseline == "on", graph=args.graph)
    import exact_io_aware_64_amd as fa
    key_groups = fa.fa_fwd_key_groups(fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32, w.B, w.H,
                                      w.N, w.n_keys, w.d, 128)
    fwd_ms = kernel_ms["fa_fwd"]
    bwd_ms = kernel_ms.get("fa_bwd")
    peak = PEAK_TFLOPS[w.dtype]
    tf_fb = (flops_f + flops_b) / (wall_ms * 1e-3) / 1e12
    tf_f = flops_f / (fwd_ms * 1e-3) / 1e12
    tf_b = flops_b / (bwd_ms * 1e-3) / 1e12 if bwd_ms else None

    # Roofline of the dominant call (largest device time per step; fa_bwd is
    # dsum_kernel then bwd_kernel, back to back on the stream): its
    # algorithmic FLOPs and compulsory bytes per call against its own
    # event-timed duration.
    kflops = kernel_flops(w.d, pairs)
    kbytes = kernel_bytes(w.B, w.H, w.N, w.d, esize, inp["seqlens"], Nk=w.n_keys)
    dom = max(kernel_ms, key=lambda n: kernel_ms[n])
    ms = kernel_ms[dom]
    t_mfma = kflops[dom] / (peak * 1e12)
    t_hbm = kbytes[dom] / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        ach = kflops[dom] / (ms * 1e-3) / 1e12
        roofline = dict(kernel=dom, bound="mfma", achieved=ach, peak=peak, unit="TFLOP/s",
                        frac=ach / peak)
    else:
        ach = kbytes[dom] / (ms * 1e-3) / 1e9
        roofline = dict(kernel=dom, bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=ach / PEAK_HBM_GBS)
    roofline.update(kernel=" + ".join(pass_kernels(w.dtype)[dom]), call=dom,
                    traffic=traffic_for(dom, key, w.dtype), flops_per_launch=kflops[dom],
                    compulsory_bytes_per_launch=kbytes[dom], launch_ms=ms)

    base = None
    parity = None
    if args.cpu_baseline == "on":
        base, parity = cpu_baseline(w, inp, outs, flops_f + flops_b, dropout_p=args.dropout)

    line = {
        "metric": METRIC,
        "value": tf_fb,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_s": args.prewarm_s,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded iid normal inputs, bf16-rounded (RNE)"
        if w.dtype == "bf16" else "synthetic: seeded iid normal fp32 inputs",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "N_k": w.n_keys, "d": w.d,
                   "causal": w.causal, "key_padding": inp["seqlens"] is not None,
                   "block_sparse": inp["block_mask"] is not None, "pairs": pairs,
                   "dropout_p": args.dropout, "step": "fwd+bwd" if w.backward else "fwd",
                   "fwd_key_groups": key_groups,
                   "step_launch": "hip graph" if args.graph else "eager"},
        "fwd_tflops": tf_f,
        "bwd_tflops": tf_b,
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "kernel_ms": kernel_ms,
        "kernel_ms_median": median_ms,
        "cold_kernel_ms": cold_ms,
        "cold_reps": args.cold_reps,
        "event_reps": max(1, args.event_reps),
        "fwd_frac_peak": tf_f / peak,
        "fwdbwd_frac_peak": tf_fb / peak,
        "peak_tflops": peak,
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "roofline": roofline,
        "cpu_baseline": base,
        "parity_sample": parity,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
