"""HIP graph capture of the attention step.  The library makes no allocation,
memset or synchronisation inside a call and launches on the caller's stream,
so a training or serving loop can record fa_fwd and fa_bwd (with its
workspace allocated beforehand), their dropout forms and fa_bwd_noalloc into
one graph through torch's stream capture and replay it.  Each test replays
the graph several times, with eager work on the same buffers in between, and
checks every replay against the eager calls bit for bit; then it copies new
inputs into the captured buffers and checks that the replay follows them."""
import sys

import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import device_inputs

pytestmark = pytest.mark.gpu

DTYPE_D = [("bf16", 64), ("bf16", 128), ("f32", 32), ("f32", 128)]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _step(fa, bufs, kw, p, ws, noalloc):
    """The calls that are recorded: forward, then backward, into bufs."""
    q, k, v, do, o, lse, dq, dk, dv = bufs
    if p > 0:
        fa.fa_fwd_dropout(q, k, v, o, lse, dropout_p=p, seed=1234, offset=7, **kw)
        fa.fa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, ws, dropout_p=p, seed=1234,
                          offset=7, **kw)
    else:
        fa.fa_fwd(q, k, v, o, lse, **kw)
        if noalloc:
            fa.fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, **kw)
        else:
            fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, **kw)


def _run(dtype, d, p, noalloc):
    import torch
    import exact_io_aware_64_amd as fa
    B, H, N = 2, 3, 700
    case = wl.random_case(B, H, N, d, dtype=dtype, seed=40 + d, causal=True, seqlens="random",
                          block_keep_p=0.7)
    q, k, v, do, sl, bm = device_inputs(case)
    kw = dict(scale=case["scale"], causal=True, seqlens_k=sl, block_mask=bm, mask_block=128)
    nb = fa.fa_bwd_workspace_bytes(1 if dtype == "f32" else 0, B, H, N, d)
    ws = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb > 0 else None
    outs = [torch.empty_like(q), torch.empty(B, H, N, device=q.device)] + \
        [torch.empty_like(q) for _ in range(3)]
    ref = [torch.empty_like(t) for t in outs]
    bufs = [q, k, v, do] + outs
    _step(fa, [q, k, v, do] + ref, kw, p, ws, noalloc)  # eager, also first-use set-up
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(fa, bufs, kw, p, ws, noalloc)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        if ws is not None:
            ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "L", "dQ", "dK", "dV"), outs, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"

    # new inputs in the captured buffers: the replay computes on them
    rng = np.random.default_rng(d + 1)
    fresh = wl.draw_tensors(rng, B, H, N, d, dtype, count=4)
    for t, x in zip((q, k, v, do), fresh):
        t.copy_(torch.from_numpy(x).to(t.dtype))
    _step(fa, [q, k, v, do] + ref, kw, p, ws, noalloc)
    torch.cuda.synchronize()
    for t in outs:
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for name, a, b in zip(("O", "L", "dQ", "dK", "dV"), outs, ref):
        assert torch.equal(a, b), f"replay on new inputs: {name} differs from the eager call"
    assert all(bool(torch.isfinite(t).all()) for t in (outs[0], outs[2], outs[3], outs[4]))


@pytest.mark.parametrize("dtype,d", DTYPE_D)
@pytest.mark.parametrize("p", [0.0, 0.1])
def test_graph_replay_equals_eager(dtype, d, p):
    _say(f"[graph] {dtype} d={d} p={p}")
    _run(dtype, d, p, noalloc=False)
    _say(f"[graph] {dtype} d={d} p={p} ok")


@pytest.mark.parametrize("dtype,d", DTYPE_D)
def test_graph_replay_noalloc(dtype, d):
    _say(f"[graph noalloc] {dtype} d={d}")
    _run(dtype, d, 0.0, noalloc=True)
    _say(f"[graph noalloc] {dtype} d={d} ok")
