"""Helpers for the GPU parity tests: move seeded numpy inputs to the device,
call the library through its binding, and measure errors against the oracle."""
from __future__ import annotations

import numpy as np

# Tolerances for the comparison with the fp64 oracle: O max-abs, L max-abs and
# relative Frobenius error of each gradient.
TOL = {
    "bf16": dict(O=1e-2, L=1e-3, G=1e-2),
    "f32": dict(O=1e-5, L=1e-5, G=1e-5),
}


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(x: np.ndarray, dtype: str, layout: str = "bhsd"):
    """fp32 numpy [B, H, N, d] -> device tensor indexed [B, H, N, d].  With
    layout "bshd" the storage is [B, N, H, d] and the result a strided view."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch_dtype(dtype))
    if layout == "bshd":
        t = t.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    else:
        t = t.contiguous().cuda()
    return t


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def opt_dev(x, dtype=None):
    import torch
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def maxabs(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nanmax(np.where(np.isnan(d), np.inf, d)))


def excess_over(o, ostar, abs_tol: float, rel: float = 2.0 ** -8) -> float:
    """Largest |o - o*| - (abs_tol + rel |o*|) over the elements (<= 0 passes):
    an absolute budget plus the rounding of the stored value, at most half
    an ulp of bf16 (2^-8 of its magnitude)."""
    o = np.asarray(o, np.float64)
    ostar = np.asarray(ostar, np.float64)
    return float(np.max(np.abs(o - ostar) - (abs_tol + rel * np.abs(ostar))))


def relfro(g, gstar) -> float:
    g = np.asarray(g, np.float64)
    gstar = np.asarray(gstar, np.float64)
    den = np.linalg.norm(gstar)
    num = np.linalg.norm(g - gstar)
    if den < 1e-12:
        return float(num)
    return float(num / den)


def device_inputs(case: dict, layout: str = "bhsd"):
    dt = case["dtype"]
    q = to_dev(case["q"], dt, layout)
    k = to_dev(case["k"], dt, layout)
    v = to_dev(case["v"], dt, layout)
    do = to_dev(case["do"], dt, layout)
    seqlens = opt_dev(case.get("seqlens"))
    bmask = opt_dev(case.get("block_mask"))
    return q, k, v, do, seqlens, bmask


def gpu_forward(case, q, k, v, seqlens, bmask):
    import exact_io_aware_64_amd as fa
    return fa.forward(q, k, v, scale=case["scale"], causal=case["causal"], seqlens_k=seqlens,
                      block_mask=bmask, mask_block=case.get("mask_block", 128))


def gpu_backward(case, q, k, v, o, do, lse, seqlens, bmask):
    import exact_io_aware_64_amd as fa
    return fa.backward(q, k, v, o, do, lse, scale=case["scale"], causal=case["causal"],
                       seqlens_k=seqlens, block_mask=bmask,
                       mask_block=case.get("mask_block", 128))


def oracle_args(case):
    return dict(scale=case["scale"], causal=case["causal"], seqlens=case.get("seqlens"),
                block_mask=case.get("block_mask"), mask_block=case.get("mask_block", 128))
