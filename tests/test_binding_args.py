"""Argument checks of the Python binding that need no GPU: every entry point
rejects key lengths, tile masks and row statistics of the wrong type, shape
or layout (and tensors off the GPU) with a ValueError before any C call, so
the kernels never receive a pointer to memory of another size or type."""
import os

import pytest
import torch

import exact_io_aware_64_amd as fa
from exact_io_aware_64_amd import _binding as bnd

pytestmark = pytest.mark.skipif(not os.path.exists(bnd.LIB_PATH),
                                reason="libfa.so not built (run __graft_entry__.build())")

B, H, N, D = 2, 3, 300, 64
NK = 520


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def _good(nk=N):
    q, o, do, dq = (_t(B, H, N, D) for _ in range(4))
    k, v, dk, dv = (_t(B, H, nk, D) for _ in range(4))
    lse = _t(B, H, N, dtype=torch.float32)
    sl = torch.tensor([N, 100], dtype=torch.int32)
    bm = torch.ones((-(-N // 128), -(-nk // 128)), dtype=torch.uint8)
    return dict(q=q, k=k, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv, lse=lse, sl=sl, bm=bm)


def _calls(t):
    """Every binding entry point with the tensors of `t` (key lengths and
    tile mask passed to all of them)."""
    kw = dict(scale=0.125, causal=True, seqlens_k=t["sl"], block_mask=t["bm"])
    qk = t["k"].shape[2] != t["q"].shape[2]
    if qk:
        return {
            "fa_fwd_qk": lambda: fa.fa_fwd_qk(t["q"], t["k"], t["v"], t["o"], t["lse"], **kw),
            "fa_bwd_qk": lambda: fa.fa_bwd_qk(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"],
                                              t["dq"], t["dk"], t["dv"], **kw),
            "prepare_fwd": lambda: fa.prepare_fwd(t["q"], t["k"], t["v"], t["o"], t["lse"], **kw),
            "prepare_bwd": lambda: fa.prepare_bwd(t["q"], t["k"], t["v"], t["o"], t["do"],
                                                  t["lse"], t["dq"], t["dk"], t["dv"], **kw),
        }
    return {
        "fa_fwd": lambda: fa.fa_fwd(t["q"], t["k"], t["v"], t["o"], t["lse"], **kw),
        "fa_fwd_tiled": lambda: fa.fa_fwd_tiled(t["q"], t["k"], t["v"], t["o"], t["lse"],
                                                block_q=128, **kw),
        "fa_fwd_dropout": lambda: fa.fa_fwd_dropout(t["q"], t["k"], t["v"], t["o"], t["lse"],
                                                    dropout_p=0.1, seed=1, **kw),
        "fa_bwd": lambda: fa.fa_bwd(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], t["dq"],
                                    t["dk"], t["dv"], **kw),
        "fa_bwd_dropout": lambda: fa.fa_bwd_dropout(t["q"], t["k"], t["v"], t["o"], t["do"],
                                                    t["lse"], t["dq"], t["dk"], t["dv"],
                                                    dropout_p=0.1, seed=1, **kw),
        "fa_bwd_dq": lambda: fa.fa_bwd_dq(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"],
                                          t["dq"], **kw),
        "fa_bwd_dkdv": lambda: fa.fa_bwd_dkdv(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"],
                                              t["dk"], t["dv"], **kw),
        "prepare_fwd": lambda: fa.prepare_fwd(t["q"], t["k"], t["v"], t["o"], t["lse"], **kw),
        "prepare_bwd": lambda: fa.prepare_bwd(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"],
                                              t["dq"], t["dk"], t["dv"], **kw),
        "prepare_fwd_tiled": lambda: fa.prepare_fwd_tiled(t["q"], t["k"], t["v"], t["o"],
                                                          t["lse"], block_q=128, **kw),
    }


BAD = {
    "seqlens int64": ("sl", lambda t: t["sl"].long(), "seqlens_k must be int32"),
    "seqlens short": ("sl", lambda t: t["sl"][:1].contiguous(), "seqlens_k must be a contiguous"),
    "seqlens strided": ("sl", lambda t: torch.zeros(2 * B, dtype=torch.int32)[::2],
                        "seqlens_k must be a contiguous"),
    "mask int32": ("bm", lambda t: t["bm"].int(), "block_mask must be uint8 or bool"),
    "mask float": ("bm", lambda t: t["bm"].float(), "block_mask must be uint8 or bool"),
    "mask too small": ("bm", lambda t: t["bm"][:-1].contiguous(),
                       "block_mask must be a contiguous"),
    "mask transposed": ("bm", lambda t: t["bm"].t(), "block_mask must be a contiguous"),
    "mask flat": ("bm", lambda t: t["bm"].reshape(-1), "block_mask must be a contiguous"),
    "lse bf16": ("lse", lambda t: t["lse"].to(torch.bfloat16), "lse must be"),
    "lse short": ("lse", lambda t: t["lse"][:, :, :-1].contiguous(), "lse must be"),
    "lse strided": ("lse", lambda t: t["lse"].transpose(0, 1).contiguous().transpose(0, 1),
                    "lse must be"),
}


@pytest.mark.parametrize("nk", [N, NK], ids=["square", "qk"])
@pytest.mark.parametrize("bad", sorted(BAD))
def test_bad_auxiliary_arguments_are_rejected(bad, nk):
    t = _good(nk)
    key, make, msg = BAD[bad]
    t[key] = make(t)
    for name, call in _calls(t).items():
        with pytest.raises(ValueError, match=msg):
            call()


@pytest.mark.parametrize("nk", [N, NK], ids=["square", "qk"])
def test_host_tensors_are_rejected(nk):
    # every argument well-formed, but in host memory
    t = _good(nk)
    for name, call in _calls(t).items():
        with pytest.raises(ValueError, match="must be on a GPU device"):
            call()


def test_bool_mask_and_no_optional_arguments_pass_the_shape_checks():
    t = _good()
    t["bm"] = t["bm"].bool()
    for name, call in _calls(t).items():
        with pytest.raises(ValueError, match="must be on a GPU device"):
            call()
    t["bm"] = None
    t["sl"] = None
    for name, call in _calls(t).items():
        with pytest.raises(ValueError, match="must be on a GPU device"):
            call()
