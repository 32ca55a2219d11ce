"""ctypes binding of libfa.so (include/fa.h).

Argument marshalling only: PyTorch tensors provide device memory, strides and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  There is no fallback: if libfa.so is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_BF16 = 0
FA_F32 = 1
FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3

# Public entry points declared in include/fa.h.
EXPORTED = ("fa_fwd", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_dq", "fa_bwd_dkdv", "fa_fwd_dropout",
            "fa_bwd_dropout", "fa_fwd_tiled", "fa_fwd_qk", "fa_bwd_qk",
            "fa_bwd_workspace_bytes", "fa_fwd_key_groups", "fa_status_string",
            "fa_last_error")


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{fa_status_string(status)}: {message}")
        self.status = status


class fa_strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("seq", ctypes.c_int64)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libfa.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} not found: build it first (python -m exact_io_aware_64_amd.build)")
    # torch brings its own HIP runtime; it has to be loaded first so that the
    # library binds to that one (loaded the other way round, the two runtimes
    # both claim the device and the first launch finds none).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, S, I, F = ctypes.c_void_p, fa_strides, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.restype = I
    lib.fa_fwd.argtypes = [I, P, S, P, S, P, S, P, S, P, I, I, I, I, F, I, P, P, I, P]
    lib.fa_bwd.restype = I
    lib.fa_bwd.argtypes = [I, P, S, P, S, P, S, P, S, P, S, P, P, S, P, S, P, S, P,
                           ctypes.c_size_t, I, I, I, I, F, I, P, P, I, P]
    lib.fa_bwd_noalloc.restype = I
    lib.fa_bwd_noalloc.argtypes = [I, P, S, P, S, P, S, P, S, P, S, P, P, S, P, S, P, S,
                                   I, I, I, I, F, I, P, P, I, P]
    lib.fa_bwd_dq.restype = I
    lib.fa_bwd_dq.argtypes = [I, P, S, P, S, P, S, P, S, P, S, P, P, S, P, ctypes.c_size_t,
                              I, I, I, I, F, I, P, P, I, P]
    lib.fa_bwd_dkdv.restype = I
    lib.fa_bwd_dkdv.argtypes = [I, P, S, P, S, P, S, P, S, P, S, P, P, S, P, S, P,
                                ctypes.c_size_t, I, I, I, I, F, I, P, P, I, P]
    U64, U32 = ctypes.c_uint64, ctypes.c_uint32
    lib.fa_fwd_qk.restype = I
    lib.fa_fwd_qk.argtypes = [I, P, S, P, S, P, S, P, S, P, I, I, I, I, I, F, I, P, P, I,
                              F, U64, U32, P]
    lib.fa_bwd_qk.restype = I
    lib.fa_bwd_qk.argtypes = [I, P, S, P, S, P, S, P, S, P, S, P, P, S, P, S, P, S, P,
                              ctypes.c_size_t, I, I, I, I, I, F, I, P, P, I, F, U64, U32, P]
    lib.fa_fwd_tiled.restype = I
    lib.fa_fwd_tiled.argtypes = [I, P, S, P, S, P, S, P, S, P, I, I, I, I, F, I, P, P, I, I, P]
    lib.fa_fwd_dropout.restype = I
    lib.fa_fwd_dropout.argtypes = [I, P, S, P, S, P, S, P, S, P, I, I, I, I, F, I, P, P, I,
                                   F, U64, U32, P]
    lib.fa_bwd_dropout.restype = I
    lib.fa_bwd_dropout.argtypes = [I, P, S, P, S, P, S, P, S, P, S, P, P, S, P, S, P, S, P,
                                   ctypes.c_size_t, I, I, I, I, F, I, P, P, I, F, U64, U32, P]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_fwd_key_groups.restype = I
    lib.fa_fwd_key_groups.argtypes = [I, I, I, I, I, I, I]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [I]
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_last_error() -> str:
    return load_library().fa_last_error().decode()


def fa_bwd_workspace_bytes(dtype: int, B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_bytes(dtype, B, H, N, d))


def fa_fwd_key_groups(dtype: int, B: int, H: int, N: int, N_k: int, d: int,
                      block_q: int = 128) -> int:
    return int(load_library().fa_fwd_key_groups(dtype, B, H, N, N_k, d, block_q))


# ------------------------------------------------------------ marshalling

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _strides(t) -> fa_strides:
    if t.dim() != 4:
        raise ValueError("expected a rank-4 tensor indexed [B, H, N, d]")
    if t.stride(3) != 1:
        raise ValueError("the last dimension must be contiguous")
    return fa_strides(t.stride(0), t.stride(1), t.stride(2))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t, stream):
    if stream is not None:
        return stream
    return _torch().cuda.current_stream(t.device).cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check(st: int):
    if st != FA_OK:
        raise FaError(st, fa_last_error())


def _workspace(q, workspace, Nq: int):
    """The backward workspace: `workspace` itself when given, else a fresh
    device buffer of fa_bwd_workspace_bytes for q's problem (None when no
    workspace is needed)."""
    if workspace is not None:
        return workspace
    B, H = q.shape[0], q.shape[1]
    try:
        code = _dtype_code(q)
    except TypeError:
        return None  # rejected later with the other arguments
    nb = fa_bwd_workspace_bytes(code, B, H, Nq, q.shape[3])
    if nb == 0 or q.device.type != "cuda":
        return None
    return _torch().empty(nb, dtype=_torch().uint8, device=q.device)


def _check_aux(q, Nq: int, Nk: int, lse, seqlens_k, block_mask, mask_block: int, tensors):
    """Checks what the library reads through raw pointers without knowing
    their types or sizes, before any C call: lse fp32 contiguous [B, H, N_q];
    seqlens_k int32 contiguous [B]; block_mask uint8 or bool contiguous
    [ceil(N_q / mask_block), ceil(N_k / mask_block)]; and every tensor
    (`tensors` are the [B, H, *, d] operands) on q's GPU."""
    torch = _torch()
    B, H = q.shape[0], q.shape[1]
    if lse is None or lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq) \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N_q] tensor")
    if seqlens_k is not None:
        if seqlens_k.dtype != torch.int32:
            raise ValueError(f"seqlens_k must be int32 (got {seqlens_k.dtype})")
        if tuple(seqlens_k.shape) != (B,) or not seqlens_k.is_contiguous():
            raise ValueError(f"seqlens_k must be a contiguous [B] = [{B}] tensor "
                             f"(got shape {tuple(seqlens_k.shape)})")
    if block_mask is not None:
        if block_mask.dtype not in (torch.uint8, torch.bool):
            raise ValueError(f"block_mask must be uint8 or bool (got {block_mask.dtype})")
        mb = int(mask_block)
        if mb <= 0:
            raise ValueError(f"mask_block must be positive (got {mb})")
        want = (-(-Nq // mb), -(-Nk // mb))
        if tuple(block_mask.shape) != want or not block_mask.is_contiguous():
            raise ValueError(f"block_mask must be a contiguous {want[0]} x {want[1]} tensor "
                             f"(got shape {tuple(block_mask.shape)})")
    if q.device.type != "cuda":
        raise ValueError(f"q must be on a GPU device (got {q.device})")
    named = [("lse", lse), ("seqlens_k", seqlens_k), ("block_mask", block_mask)]
    for name, t in list(tensors) + named:
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} must be on {q.device} like q (got {t.device})")


def _fwd_args(q, k, v, o, lse, scale, causal, seqlens_k, block_mask, mask_block):
    B, H, N, d = _check_like(q, (("k", k), ("v", v), ("o", o)))
    _check_aux(q, N, N, lse, seqlens_k, block_mask, mask_block,
               (("k", k), ("v", v), ("o", o)))
    return (_dtype_code(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
            _ptr(o), _strides(o), _ptr(lse), B, H, N, d, float(scale), int(bool(causal)),
            _ptr(seqlens_k), _ptr(block_mask), int(mask_block))


def _check_qk(q, k, qside, kside):
    """Shapes [B, H, N_q, d] (q and qside) and [B, H, N_k, d] (k and kside),
    one dtype; returns B, H, N_q, N_k, d."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for name, t in qside:
        if tuple(t.shape) != (B, H, Nq, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [B, H, N_q, d] like q")
    for name, t in (("k", k),) + tuple(kside):
        if tuple(t.shape) != (B, H, Nk, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [B, H, N_k, d] like k")
    return B, H, Nq, Nk, d


def fa_fwd_qk(q, k, v, o, lse, *, scale: float, causal: bool = False, seqlens_k=None,
              block_mask=None, mask_block: int = 128, dropout_p: float = 0.0, seed: int = 0,
              offset: int = 0, stream=None) -> None:
    """Calls fa_fwd_qk: q, o [B, H, N_q, d]; k, v [B, H, N_k, d]; causal keys
    j <= i + N_k - N_q."""
    lib = load_library()
    B, H, Nq, Nk, d = _check_qk(q, k, (("o", o),), (("v", v),))
    _check_aux(q, Nq, Nk, lse, seqlens_k, block_mask, mask_block,
               (("k", k), ("v", v), ("o", o)))
    st = lib.fa_fwd_qk(_dtype_code(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                       _strides(v), _ptr(o), _strides(o), _ptr(lse), B, H, Nq, Nk, d,
                       float(scale), int(bool(causal)), _ptr(seqlens_k), _ptr(block_mask),
                       int(mask_block), *_drop_args(dropout_p, seed, offset), _stream(q, stream))
    _check(st)


def fa_bwd_qk(q, k, v, o, dout, lse, dq, dk, dv, workspace=None, *, scale: float,
              causal: bool = False, seqlens_k=None, block_mask=None, mask_block: int = 128,
              dropout_p: float = 0.0, seed: int = 0, offset: int = 0, stream=None) -> None:
    """Calls fa_bwd_qk (the forward call's lengths, masks and dropout).  A
    workspace is allocated when none is given."""
    lib = load_library()
    B, H, Nq, Nk, d = _check_qk(q, k, (("o", o), ("dout", dout), ("dq", dq)),
                                (("v", v), ("dk", dk), ("dv", dv)))
    workspace = _workspace(q, workspace, Nq)
    _check_aux(q, Nq, Nk, lse, seqlens_k, block_mask, mask_block,
               (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk),
                ("dv", dv), ("workspace", workspace)))
    st = lib.fa_bwd_qk(_dtype_code(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                       _strides(v), _ptr(o), _strides(o), _ptr(dout), _strides(dout), _ptr(lse),
                       _ptr(dq), _strides(dq), _ptr(dk), _strides(dk), _ptr(dv), _strides(dv),
                       _ptr(workspace), _nbytes(workspace), B, H, Nq, Nk, d, float(scale),
                       int(bool(causal)), _ptr(seqlens_k), _ptr(block_mask), int(mask_block),
                       *_drop_args(dropout_p, seed, offset), _stream(q, stream))
    _check(st)


def _drop_args(dropout_p, seed, offset):
    return (float(dropout_p), int(seed) & (2**64 - 1), int(offset) & (2**32 - 1))


def fa_fwd(q, k, v, o, lse, *, scale: float, causal: bool = False, seqlens_k=None,
           block_mask=None, mask_block: int = 128, stream=None) -> None:
    """Calls fa_fwd on tensors indexed [B, H, N, d] (any strides with a
    contiguous last dimension); o and lse ([B, H, N] fp32, contiguous) are
    written."""
    lib = load_library()
    args = _fwd_args(q, k, v, o, lse, scale, causal, seqlens_k, block_mask, mask_block)
    _check(lib.fa_fwd(*args, _stream(q, stream)))


def fa_fwd_tiled(q, k, v, o, lse, *, scale: float, block_q: int, causal: bool = False,
                 seqlens_k=None, block_mask=None, mask_block: int = 128, stream=None) -> None:
    """Calls fa_fwd_tiled (fa_fwd with block_q query rows per workgroup)."""
    lib = load_library()
    args = _fwd_args(q, k, v, o, lse, scale, causal, seqlens_k, block_mask, mask_block)
    _check(lib.fa_fwd_tiled(*args, int(block_q), _stream(q, stream)))


def prepare_fwd_tiled(q, k, v, o, lse, *, scale: float, block_q: int, causal: bool = False,
                      seqlens_k=None, block_mask=None, mask_block: int = 128,
                      stream=None) -> "Prepared":
    """fa_fwd_tiled with fixed arguments."""
    lib = load_library()
    args = _fwd_args(q, k, v, o, lse, scale, causal, seqlens_k, block_mask, mask_block)
    return Prepared(lib.fa_fwd_tiled, args + (int(block_q), _stream(q, stream)),
                    (q, k, v, o, lse, seqlens_k, block_mask))


def fa_fwd_dropout(q, k, v, o, lse, *, scale: float, dropout_p: float, seed: int,
                   offset: int = 0, causal: bool = False, seqlens_k=None, block_mask=None,
                   mask_block: int = 128, stream=None) -> None:
    """Calls fa_fwd_dropout (fa_fwd with dropout on the probabilities)."""
    lib = load_library()
    args = _fwd_args(q, k, v, o, lse, scale, causal, seqlens_k, block_mask, mask_block)
    _check(lib.fa_fwd_dropout(*args, *_drop_args(dropout_p, seed, offset), _stream(q, stream)))


def _check_like(q, named):
    B, H, N, d = q.shape
    for name, t in named:
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    return B, H, N, d


def _bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal, seqlens_k,
              block_mask, mask_block):
    named = (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv))
    B, H, N, d = _check_like(q, named)
    workspace = _workspace(q, workspace, N)
    _check_aux(q, N, N, lse, seqlens_k, block_mask, mask_block,
               named + (("workspace", workspace),))
    return (_dtype_code(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
            _ptr(o), _strides(o), _ptr(dout), _strides(dout), _ptr(lse), _ptr(dq), _strides(dq),
            _ptr(dk), _strides(dk), _ptr(dv), _strides(dv), _ptr(workspace), _nbytes(workspace),
            B, H, N, d, float(scale), int(bool(causal)), _ptr(seqlens_k), _ptr(block_mask),
            int(mask_block))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace=None, *, scale: float,
           causal: bool = False, seqlens_k=None, block_mask=None, mask_block: int = 128,
           stream=None) -> None:
    """Calls fa_bwd; dq, dk, dv are written in full.  A workspace of
    fa_bwd_workspace_bytes is allocated when none is given."""
    lib = load_library()
    args = _bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal, seqlens_k,
                     block_mask, mask_block)
    _check(lib.fa_bwd(*args, _stream(q, stream)))


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, *, scale: float, causal: bool = False,
                   seqlens_k=None, block_mask=None, mask_block: int = 128,
                   stream=None) -> None:
    """Calls fa_bwd_noalloc: fa_bwd with D in the library's own scratch array
    (no workspace; calls that overlap on one GPU race)."""
    lib = load_library()
    named = (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv))
    B, H, N, d = _check_like(q, named)
    _check_aux(q, N, N, lse, seqlens_k, block_mask, mask_block, named)
    st = lib.fa_bwd_noalloc(_dtype_code(q), _ptr(q), _strides(q), _ptr(k), _strides(k),
                            _ptr(v), _strides(v), _ptr(o), _strides(o), _ptr(dout),
                            _strides(dout), _ptr(lse), _ptr(dq), _strides(dq), _ptr(dk),
                            _strides(dk), _ptr(dv), _strides(dv), B, H, N, d, float(scale),
                            int(bool(causal)), _ptr(seqlens_k), _ptr(block_mask),
                            int(mask_block), _stream(q, stream))
    _check(st)


def fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, workspace=None, *, scale: float,
                   dropout_p: float, seed: int, offset: int = 0, causal: bool = False,
                   seqlens_k=None, block_mask=None, mask_block: int = 128,
                   stream=None) -> None:
    """Calls fa_bwd_dropout; needs the forward call's dropout_p, seed and offset."""
    lib = load_library()
    args = _bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal, seqlens_k,
                     block_mask, mask_block)
    _check(lib.fa_bwd_dropout(*args, *_drop_args(dropout_p, seed, offset), _stream(q, stream)))


def fa_bwd_dq(q, k, v, o, dout, lse, dq, workspace=None, *, scale: float,
              causal: bool = False, seqlens_k=None, block_mask=None, mask_block: int = 128,
              stream=None) -> None:
    """Calls fa_bwd_dq: writes dq in full."""
    lib = load_library()
    named = (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq))
    B, H, N, d = _check_like(q, named)
    workspace = _workspace(q, workspace, N)
    _check_aux(q, N, N, lse, seqlens_k, block_mask, mask_block,
               named + (("workspace", workspace),))
    nbytes = _nbytes(workspace)
    st = lib.fa_bwd_dq(_dtype_code(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                       _strides(v), _ptr(o), _strides(o), _ptr(dout), _strides(dout),
                       _ptr(lse), _ptr(dq), _strides(dq), _ptr(workspace), nbytes, B, H, N, d,
                       float(scale), int(bool(causal)), _ptr(seqlens_k), _ptr(block_mask),
                       int(mask_block), _stream(q, stream))
    _check(st)


def fa_bwd_dkdv(q, k, v, o, dout, lse, dk, dv, workspace=None, *, scale: float,
                causal: bool = False, seqlens_k=None, block_mask=None, mask_block: int = 128,
                stream=None) -> None:
    """Calls fa_bwd_dkdv: writes dk and dv in full."""
    lib = load_library()
    named = (("k", k), ("v", v), ("o", o), ("dout", dout), ("dk", dk), ("dv", dv))
    B, H, N, d = _check_like(q, named)
    workspace = _workspace(q, workspace, N)
    _check_aux(q, N, N, lse, seqlens_k, block_mask, mask_block,
               named + (("workspace", workspace),))
    nbytes = _nbytes(workspace)
    st = lib.fa_bwd_dkdv(_dtype_code(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                         _strides(v), _ptr(o), _strides(o), _ptr(dout), _strides(dout),
                         _ptr(lse), _ptr(dk),
                         _strides(dk), _ptr(dv), _strides(dv), _ptr(workspace), nbytes, B, H,
                         N, d, float(scale), int(bool(causal)), _ptr(seqlens_k),
                         _ptr(block_mask), int(mask_block), _stream(q, stream))
    _check(st)


# ---------------------------------------------------------- prepared calls

class Prepared:
    """One C-ABI call with every argument converted once: calling it costs a
    single ctypes call, so a tight loop of launches is not held back by the
    host.  Tensors must stay alive (and keep their storage) while it is used."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep  # the tensors whose pointers are baked into args

    def __call__(self) -> None:
        _check(self._fn(*self._args))


def prepare_fwd(q, k, v, o, lse, *, scale: float, causal: bool = False, seqlens_k=None,
                block_mask=None, mask_block: int = 128, dropout_p: float = 0.0, seed: int = 0,
                offset: int = 0, stream=None) -> Prepared:
    """fa_fwd (or fa_fwd_dropout when dropout_p > 0, fa_fwd_qk when k has
    another length) with fixed arguments."""
    lib = load_library()
    keep = (q, k, v, o, lse, seqlens_k, block_mask)
    if k.shape[2] != q.shape[2]:
        B, H, Nq, Nk, d = _check_qk(q, k, (("o", o),), (("v", v),))
        _check_aux(q, Nq, Nk, lse, seqlens_k, block_mask, mask_block,
                   (("k", k), ("v", v), ("o", o)))
        args = (_dtype_code(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                _strides(v), _ptr(o), _strides(o), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                int(bool(causal)), _ptr(seqlens_k), _ptr(block_mask), int(mask_block))
        return Prepared(lib.fa_fwd_qk,
                        args + _drop_args(dropout_p, seed, offset) + (_stream(q, stream),), keep)
    args = _fwd_args(q, k, v, o, lse, scale, causal, seqlens_k, block_mask, mask_block)
    if dropout_p > 0:
        return Prepared(lib.fa_fwd_dropout,
                        args + _drop_args(dropout_p, seed, offset) + (_stream(q, stream),), keep)
    return Prepared(lib.fa_fwd, args + (_stream(q, stream),), keep)


def prepare_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace=None, *, scale: float,
                causal: bool = False, seqlens_k=None, block_mask=None, mask_block: int = 128,
                dropout_p: float = 0.0, seed: int = 0, offset: int = 0,
                stream=None) -> Prepared:
    """fa_bwd (or fa_bwd_dropout when dropout_p > 0, fa_bwd_qk when k has
    another length) with fixed arguments."""
    lib = load_library()
    workspace = _workspace(q, workspace, q.shape[2])
    keep = (q, k, v, o, dout, lse, dq, dk, dv, workspace, seqlens_k, block_mask)
    if k.shape[2] != q.shape[2]:
        B, H, Nq, Nk, d = _check_qk(q, k, (("o", o), ("dout", dout), ("dq", dq)),
                                    (("v", v), ("dk", dk), ("dv", dv)))
        _check_aux(q, Nq, Nk, lse, seqlens_k, block_mask, mask_block,
                   (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv), ("workspace", workspace)))
        args = (_dtype_code(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                _strides(v), _ptr(o), _strides(o), _ptr(dout), _strides(dout), _ptr(lse),
                _ptr(dq), _strides(dq), _ptr(dk), _strides(dk), _ptr(dv), _strides(dv),
                _ptr(workspace), _nbytes(workspace), B, H, Nq, Nk, d, float(scale),
                int(bool(causal)), _ptr(seqlens_k), _ptr(block_mask), int(mask_block))
        return Prepared(lib.fa_bwd_qk,
                        args + _drop_args(dropout_p, seed, offset) + (_stream(q, stream),), keep)
    args = _bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, causal, seqlens_k,
                     block_mask, mask_block)
    if dropout_p > 0:
        return Prepared(lib.fa_bwd_dropout,
                        args + _drop_args(dropout_p, seed, offset) + (_stream(q, stream),), keep)
    return Prepared(lib.fa_bwd, args + (_stream(q, stream),), keep)


# --------------------------------------------- allocating convenience calls

def forward(q, k, v, *, scale: float, causal: bool = False, seqlens_k=None, block_mask=None,
            mask_block: int = 128, dropout_p: float = 0.0, seed: int = 0, offset: int = 0):
    """Allocates O (contiguous [B, H, N, d]) and L, then calls fa_fwd (or
    fa_fwd_dropout when dropout_p > 0, fa_fwd_qk when k has another length)."""
    torch = _torch()
    B, H, N, d = q.shape
    o = torch.empty((B, H, N, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    kw = dict(scale=scale, causal=causal, seqlens_k=seqlens_k, block_mask=block_mask,
              mask_block=mask_block)
    if k.shape[2] != N:
        fa_fwd_qk(q, k, v, o, lse, dropout_p=dropout_p, seed=seed, offset=offset, **kw)
    elif dropout_p > 0:
        fa_fwd_dropout(q, k, v, o, lse, dropout_p=dropout_p, seed=seed, offset=offset, **kw)
    else:
        fa_fwd(q, k, v, o, lse, **kw)
    return o, lse


def backward(q, k, v, o, dout, lse, *, scale: float, causal: bool = False, seqlens_k=None,
             block_mask=None, mask_block: int = 128, workspace=None, dropout_p: float = 0.0,
             seed: int = 0, offset: int = 0):
    """Allocates dQ, dK, dV (and the workspace unless given), then calls fa_bwd
    (or fa_bwd_dropout when dropout_p > 0, fa_bwd_qk when k has another length)."""
    torch = _torch()
    B, H, N, d = q.shape
    Nk = k.shape[2]
    dq = torch.empty((B, H, N, d), dtype=q.dtype, device=q.device)
    dk = torch.empty((B, H, Nk, d), dtype=q.dtype, device=q.device)
    dv = torch.empty_like(dk)
    workspace = _workspace(q, workspace, N)
    kw = dict(scale=scale, causal=causal, seqlens_k=seqlens_k, block_mask=block_mask,
              mask_block=mask_block)
    if Nk != N:
        fa_bwd_qk(q, k, v, o, dout, lse, dq, dk, dv, workspace, dropout_p=dropout_p,
                  seed=seed, offset=offset, **kw)
    elif dropout_p > 0:
        fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, workspace, dropout_p=dropout_p,
                       seed=seed, offset=offset, **kw)
    else:
        fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, **kw)
    return dq, dk, dv


# Short names of the two allocating calls: fwd(q, k, v, ...) -> (o, lse) and
# bwd(q, k, v, o, dout, lse, ...) -> (dq, dk, dv).
fwd = forward
bwd = backward
