#!/usr/bin/env python3
"""Attention throughput on one MI355X.

One step = the whole hot path on one batch: fa_fwd (scores, mask, online
softmax, O and L) followed by fa_bwd (D, dQ, dK, dV recomputed from L).
Prints one JSON line with forward+backward TFLOP/s (the value), forward
TFLOP/s, both as fractions of the bf16 dense MFMA peak, a roofline entry for
the dominant kernel and the fp64 CPU oracle timed on the host as a baseline.

FLOP convention (algorithmic work over visible (query, key) pairs; masked-out
tiles are never credited): forward 4*d*pairs, backward 10*d*pairs.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--cpu-baseline off]
"""
from __future__ import annotations

import argparse
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
DEFAULT_WORKLOAD = "gpt2s_causal_b8h12n1024"


# --------------------------------------------------------------- accounting

def visible_pairs(N: int, H: int, causal: bool, seqlens, block_mask, mask_block: int = 128,
                  B: int = 1) -> int:
    """Number of visible (query, key) pairs summed over batch and heads."""
    lens = [N] * B if seqlens is None else [int(min(max(s, 0), N)) for s in seqlens]
    total = 0
    for L in lens:
        if block_mask is None:
            if causal:
                total += L * (L + 1) // 2 + (N - L) * L
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
                total += int(np.clip(np.minimum(i + 1, e) - c, 0, None).sum())
    return total * H


def kernel_bytes(B, H, N, d, esize, seqlens):
    """Compulsory HBM bytes per launch of each kernel: every tensor the kernel
    must read or write once (keys and values only up to each sequence's key
    length), plus the fp32 row statistics L and D."""
    t = B * H * N * d * esize
    kv_valid = H * d * esize * (B * N if seqlens is None else int(np.minimum(seqlens, N).sum()))
    rowstat = B * H * N * 4
    return {
        "fwd_bf16_kernel": 2 * t + 2 * kv_valid + rowstat,         # Q, O; K, V; L
        "dq_kernel": 4 * t + 2 * kv_valid + 2 * rowstat,           # Q, O, dO, dQ; K, V; L, D
        "dkdv_kernel": 4 * t + 2 * kv_valid + 2 * rowstat,         # Q, dO, dK, dV; K, V; L, D
    }


def kernel_flops(d, pairs):
    """Algorithmic FLOPs per launch.  The method's backward pass is five
    products over visible pairs (S recomputed, dV, dP, dQ, dK; 2*d each): the
    dK/dV kernel performs four of them, the dQ kernel the fifth (its own
    recomputation of S and dP duplicates work and is not credited)."""
    return {"fwd_bf16_kernel": 4.0 * d * pairs, "dq_kernel": 2.0 * d * pairs,
            "dkdv_kernel": 8.0 * d * pairs}


# ------------------------------------------------------------------- timing

KERNELS = ("fwd_bf16_kernel", "dq_kernel", "dkdv_kernel")


def run_gpu(w: wl.Workload, inp: dict, steps: int, warmup: int):
    """Times `steps` steps after `warmup` untimed ones.  One step is fa_fwd,
    then the two phases of the backward pass (fa_bwd_dq, fa_bwd_dkdv), each a
    single kernel launch on the current stream; HIP events recorded on that
    stream between the launches give each kernel's device time, and the wall
    clock around the whole timed region gives the step time."""
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
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32
    ws = torch.empty(fa.fa_bwd_workspace_bytes(code, w.B, w.H, w.N, w.d), dtype=torch.uint8,
                     device=dev)
    kw = dict(scale=w.scale, causal=w.causal, seqlens_k=sl, block_mask=bm, mask_block=128)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fa_fwd(q, k, v, o, lse, **kw)
        if ev is not None:
            ev[1].record(stream)
        fa.fa_bwd_dq(q, k, v, o, do, lse, dq, ws, **kw)
        if ev is not None:
            ev[2].record(stream)
        fa.fa_bwd_dkdv(q, k, v, do, lse, dk, dv, ws, **kw)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    kernel_ms = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
                 for i, name in enumerate(KERNELS)}
    props = torch.cuda.get_device_properties(dev)
    outs = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
    return wall_ms, kernel_ms, props, outs


def cpu_baseline(w: wl.Workload, inp: dict, outs: dict, flops_fb: float,
                 budget_s: float = 10.0):
    """The fp64 oracle as it stands, on the host cores, on the same inputs.

    Sample: whole (batch, head) slices of the workload -- all heads when one
    pass fits the budget, else the first heads -- repeated until about
    ``budget_s`` seconds of CPU work; the value is scaled by the FLOPs of what
    was computed."""
    from oracle import attention_ref as ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    args = dict(scale=w.scale, causal=w.causal, seqlens=inp["seqlens"],
                block_mask=inp["block_mask"], mask_block=128)
    H = w.H
    sub = lambda x, hs: x[:, :hs]  # noqa: E731

    def one_pass(hs):
        O, L = ref.forward(sub(inp["q"], hs), sub(inp["k"], hs), sub(inp["v"], hs), **args)
        G = ref.backward(sub(inp["q"], hs), sub(inp["k"], hs), sub(inp["v"], hs),
                         sub(inp["do"], hs), **args)
        return O, L, G

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
    tflops = flops_fb * (hs / H) * passes / secs / 1e12
    # the same sample doubles as a parity spot check of the GPU outputs
    npf = lambda t: t[:, :hs].float().cpu().numpy().astype(np.float64)  # noqa: E731
    lg = npf(outs["lse"])
    fin = np.isfinite(L)
    parity = dict(O_maxabs=float(np.abs(npf(outs["o"]) - O).max()),
                  L_maxabs=float(np.abs(lg[fin] - L[fin]).max()) if fin.any() else 0.0)
    for name, g in zip(("dQ", "dK", "dV"), G):
        parity[f"{name}_relfro"] = float(np.linalg.norm(npf(outs["d" + name[1].lower()]) - g)
                                         / np.linalg.norm(g))
    base = dict(value=tflops, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"fp64 NumPy oracle fwd+bwd on {hs} of {H} heads x batch {w.B} "
                       f"(whole sequences), {passes} pass(es) in {secs:.1f} s; value scaled "
                       f"by the FLOPs of the sample",
                seconds=secs)
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


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=wl.WORKLOAD_ORDER)
    ap.add_argument("--cpu-baseline", default="on", choices=["on", "off"])
    ap.add_argument("--mode", default="attention", choices=["attention", "copy"],
                    help="copy: time a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--copy-mib", type=int, default=1024)
    args = ap.parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the attention path needs no collective and "
              "this build runs on a single MI355X (heads shard across GPUs with no "
              "communication). Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.mode == "copy":
        return copy_calibration(args.copy_mib, args.steps, args.warmup)

    w = wl.WORKLOADS[args.workload]
    inp = wl.make_inputs(w)
    pairs = visible_pairs(w.N, w.H, w.causal, inp["seqlens"], inp["block_mask"], 128, w.B)
    flops_f = 4.0 * w.d * pairs
    flops_b = 10.0 * w.d * pairs
    esize = 2 if w.dtype == "bf16" else 4

    wall_ms, kernel_ms, props, outs = run_gpu(w, inp, args.steps, args.warmup)
    fwd_ms = kernel_ms["fwd_bf16_kernel"]
    bwd_ms = kernel_ms["dq_kernel"] + kernel_ms["dkdv_kernel"]
    peak = PEAK_TFLOPS[w.dtype]
    tf_fb = (flops_f + flops_b) / (wall_ms * 1e-3) / 1e12
    tf_f = flops_f / (fwd_ms * 1e-3) / 1e12
    tf_b = flops_b / (bwd_ms * 1e-3) / 1e12

    # Roofline of the dominant kernel (largest device time per step): its
    # algorithmic FLOPs and compulsory bytes per launch against its own
    # event-timed duration.
    kflops = kernel_flops(w.d, pairs)
    kbytes = kernel_bytes(w.B, w.H, w.N, w.d, esize, inp["seqlens"])
    dom = max(KERNELS, key=lambda n: kernel_ms[n])
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
    roofline.update(traffic=None, flops_per_launch=kflops[dom],
                    compulsory_bytes_per_launch=kbytes[dom], launch_ms=ms)

    base = None
    parity = None
    if args.cpu_baseline == "on":
        base, parity = cpu_baseline(w, inp, outs, flops_f + flops_b)

    line = {
        "metric": METRIC,
        "value": tf_fb,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded iid normal inputs, bf16-rounded (RNE)"
        if w.dtype == "bf16" else "synthetic: seeded iid normal fp32 inputs",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "key_padding": inp["seqlens"] is not None,
                   "block_sparse": inp["block_mask"] is not None, "pairs": pairs},
        "fwd_tflops": tf_f,
        "bwd_tflops": tf_b,
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "kernel_ms": kernel_ms,
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
