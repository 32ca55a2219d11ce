"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/fa.h, and rejects bad arguments on the host before any
HIP call (so these calls never launch anything)."""
import ctypes
import os
import re

import pytest

import exact_io_aware_64_amd as fa
from exact_io_aware_64_amd import _binding as bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(bnd.LIB_PATH),
                                reason="libfa.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(fa.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bnd.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert fa.fa_status_string(0) == "FA_OK"
    assert fa.fa_status_string(1) == "FA_ERR_INVALID_ARG"
    assert fa.fa_status_string(2) == "FA_ERR_UNSUPPORTED"
    assert fa.fa_status_string(3) == "FA_ERR_HIP"
    assert fa.fa_status_string(99) == "FA_UNKNOWN_STATUS"


def test_workspace_bytes():
    # bf16: one fp32 D per query row, rounded up to 256 bytes; fp32 kernels
    # keep D on chip
    assert fa.fa_bwd_workspace_bytes(0, 8, 12, 1024, 64) == 8 * 12 * 1024 * 4
    assert fa.fa_bwd_workspace_bytes(0, 1, 8, 65536, 64) == 8 * 65536 * 4
    assert fa.fa_bwd_workspace_bytes(0, 1, 1, 3, 128) == 256
    assert fa.fa_bwd_workspace_bytes(0, 2, 3, 100, 32) == 2560
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 3, 64) == 0
    assert fa.fa_bwd_workspace_bytes(0, 0, 1, 3, 64) == 0


def test_key_groups_without_device_query():
    # cases decided before the device's CU count is read: no split
    assert fa.fa_fwd_key_groups(fa.FA_F32, 1, 1, 4096, 4096, 64, 128) == 1
    assert fa.fa_fwd_key_groups(fa.FA_BF16, 1, 1, 4096, 4096, 64, 64) == 1
    assert fa.fa_fwd_key_groups(fa.FA_BF16, 1, 1, 4096, 1023, 64, 128) == 1
    assert fa.fa_fwd_key_groups(fa.FA_BF16, 0, 1, 4096, 4096, 64, 128) == 1


# Fake, suitably aligned device addresses: every call below must be rejected
# by host-side validation, so they are never dereferenced.
A = 0x10000
S = bnd.fa_strides(8 * 1024 * 64, 1024 * 64, 64)


def _fwd(**kw):
    lib = fa.load_library()
    args = dict(dtype=0, q=A, sq=S, k=A, sk=S, v=A, sv=S, o=A, so=S, lse=A, B=1, H=1, N=1024,
                d=64, scale=0.125, causal=1, seqlens=None, bmask=None, mb=128, stream=None)
    args.update(kw)
    return lib.fa_fwd(*args.values())


def _bwd(**kw):
    lib = fa.load_library()
    args = dict(dtype=0, q=A, sq=S, k=A, sk=S, v=A, sv=S, o=A, so=S, do=A, sdo=S, lse=A,
                dq=A, sdq=S, dk=A, sdk=S, dv=A, sdv=S, ws=A, wsb=4096, B=1, H=1, N=1024,
                d=64, scale=0.125, causal=0, seqlens=None, bmask=None, mb=128, stream=None)
    args.update(kw)
    return lib.fa_bwd(*args.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=None), 1, "q is NULL"),
    (dict(lse=None), 1, "lse is NULL"),
    (dict(v=A + 8), 1, "v is not 16-byte aligned"),
    (dict(B=0), 1, "must be positive"),
    (dict(N=-5), 1, "must be positive"),
    (dict(d=96), 2, "head dimension"),
    (dict(d=96, dtype=1), 2, "head dimension"),
    (dict(d=256, dtype=1), 2, "head dimension"),
    (dict(scale=0.0), 1, "scale"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(dtype=7), 1, "dtype"),
    (dict(sk=bnd.fa_strides(64, 64, 60)), 1, "multiples of 8"),
    (dict(so=bnd.fa_strides(-64, 64, 64)), 1, "negative"),
    (dict(bmask=A, mb=64), 1, "mask_block"),
    (dict(bmask=A, mb=100), 1, "mask_block"),
    (dict(bmask=A, N=300000), 2, "block mask"),
    (dict(seqlens=A + 2), 1, "seqlens_k"),
    (dict(sq=bnd.fa_strides(0, 0, 1 << 20), N=1024), 2, "2 GiB"),
])
def test_fwd_rejects_bad_arguments(kw, status, msg):
    assert _fwd(**kw) == status
    assert msg in fa.fa_last_error()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dq=None), 1, "dq is NULL"),
    (dict(o=None), 1, "o is NULL"),
    (dict(do=A + 4), 1, "dout is not 16-byte aligned"),
    (dict(dtype=1, sdv=bnd.fa_strides(64, 64, 66)), 1, "multiples of 4"),
    (dict(d=96), 2, "head dimension"),
    (dict(d=96, dtype=1), 2, "head dimension"),
    (dict(ws=None, wsb=0), 1, "workspace is NULL"),
    (dict(wsb=4095), 1, "workspace too small"),
    (dict(ws=A + 8), 1, "workspace is not 16-byte aligned"),
    (dict(B=2, wsb=4096), 1, "workspace too small"),
])
def test_bwd_rejects_bad_arguments(kw, status, msg):
    assert _bwd(**kw) == status
    assert msg in fa.fa_last_error()


def _bwd_dq(**kw):
    lib = fa.load_library()
    args = dict(dtype=0, q=A, sq=S, k=A, sk=S, v=A, sv=S, o=A, so=S, do=A, sdo=S, lse=A,
                dq=A, sdq=S, ws=A, wsb=4096, B=1, H=1, N=1024, d=64, scale=0.125, causal=0,
                seqlens=None, bmask=None, mb=128, stream=None)
    args.update(kw)
    return lib.fa_bwd_dq(*args.values())


def _bwd_dkdv(**kw):
    lib = fa.load_library()
    args = dict(dtype=0, q=A, sq=S, k=A, sk=S, v=A, sv=S, o=A, so=S, do=A, sdo=S, lse=A, dk=A,
                sdk=S,
                dv=A, sdv=S, ws=A, wsb=4096, B=1, H=1, N=1024, d=64, scale=0.125, causal=0,
                seqlens=None, bmask=None, mb=128, stream=None)
    args.update(kw)
    return lib.fa_bwd_dkdv(*args.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dq=None), 1, "dq is NULL"),
    (dict(o=A + 4), 1, "o is not 16-byte aligned"),
    (dict(lse=None), 1, "lse is NULL"),
    (dict(N=0), 1, "must be positive"),
    (dict(ws=None, wsb=0), 1, "workspace is NULL"),
])
def test_bwd_dq_rejects_bad_arguments(kw, status, msg):
    assert _bwd_dq(**kw) == status
    assert msg in fa.fa_last_error()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dk=None), 1, "dk is NULL"),
    (dict(dv=A + 2), 1, "dv is not 16-byte aligned"),
    (dict(o=None), 1, "o is NULL"),
    (dict(do=None), 1, "dout is NULL"),
    (dict(d=96), 2, "head dimension"),
    (dict(d=256, dtype=1), 2, "head dimension"),
    (dict(wsb=1024), 1, "workspace too small"),
])
def test_bwd_dkdv_rejects_bad_arguments(kw, status, msg):
    assert _bwd_dkdv(**kw) == status
    assert msg in fa.fa_last_error()


def test_missing_library_raises(tmp_path):
    with pytest.raises(RuntimeError, match="not found"):
        _load_fresh(str(tmp_path / "nope.so"))


def _load_fresh(path):
    saved = bnd._lib
    bnd._lib = None
    try:
        return bnd.load_library(path)
    finally:
        bnd._lib = saved


def _fwd_drop(**kw):
    lib = fa.load_library()
    args = dict(dtype=0, q=A, sq=S, k=A, sk=S, v=A, sv=S, o=A, so=S, lse=A, B=1, H=1, N=1024,
                d=64, scale=0.125, causal=1, seqlens=None, bmask=None, mb=128, p=0.1, seed=1,
                offset=0, stream=None)
    args.update(kw)
    return lib.fa_fwd_dropout(*args.values())


def _bwd_drop(**kw):
    lib = fa.load_library()
    args = dict(dtype=0, q=A, sq=S, k=A, sk=S, v=A, sv=S, o=A, so=S, do=A, sdo=S, lse=A,
                dq=A, sdq=S, dk=A, sdk=S, dv=A, sdv=S, ws=A, wsb=4096, B=1, H=1, N=1024,
                d=64, scale=0.125, causal=0, seqlens=None, bmask=None, mb=128, p=0.1, seed=1,
                offset=0, stream=None)
    args.update(kw)
    return lib.fa_bwd_dropout(*args.values())


BAD_DROPOUT = [
    (dict(p=1.0), 1, "dropout_p must lie in [0, 1)"),
    (dict(p=-0.1), 1, "dropout_p must lie in [0, 1)"),
    (dict(p=float("nan")), 1, "dropout_p must lie in [0, 1)"),
    (dict(p=0.999), 1, "rounds to dropping every pair"),
    (dict(p=0.1, q=None), 1, "q is NULL"),
    (dict(p=0.1, d=96), 2, "head dimension"),
    (dict(p=0.1, d=96, dtype=1), 2, "head dimension"),
    (dict(p=0.1, d=256, dtype=1), 2, "head dimension"),
]


@pytest.mark.parametrize("kw,status,msg", BAD_DROPOUT)
def test_fwd_dropout_rejects_bad_arguments(kw, status, msg):
    assert _fwd_drop(**kw) == status
    assert msg in fa.fa_last_error()


@pytest.mark.parametrize("kw,status,msg", BAD_DROPOUT + [(dict(dq=None), 1, "dq is NULL")])
def test_bwd_dropout_rejects_bad_arguments(kw, status, msg):
    assert _bwd_drop(**kw) == status
    assert msg in fa.fa_last_error()


def _fwd_tiled(**kw):
    lib = fa.load_library()
    args = dict(dtype=0, q=A, sq=S, k=A, sk=S, v=A, sv=S, o=A, so=S, lse=A, B=1, H=1, N=1024,
                d=64, scale=0.125, causal=1, seqlens=None, bmask=None, mb=128, bq=64,
                stream=None)
    args.update(kw)
    return lib.fa_fwd_tiled(*args.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(bq=100), 1, "block_q must be 64, 128 or 256"),
    (dict(bq=32), 1, "block_q must be 64, 128 or 256"),
    (dict(bq=64, dtype=1), 2, "bf16 only"),
    (dict(bq=256, bmask=A, mb=128), 2, "does not divide mask_block"),
    (dict(bq=256, q=None), 1, "q is NULL"),
])
def test_fwd_tiled_rejects_bad_arguments(kw, status, msg):
    assert _fwd_tiled(**kw) == status
    assert msg in fa.fa_last_error()


def _fwd_qk(**kw):
    lib = fa.load_library()
    args = dict(dtype=0, q=A, sq=S, k=A, sk=S, v=A, sv=S, o=A, so=S, lse=A, B=1, H=1, Nq=16,
                Nk=1024, d=64, scale=0.125, causal=1, seqlens=None, bmask=None, mb=128, p=0.0,
                seed=0, offset=0, stream=None)
    args.update(kw)
    return lib.fa_fwd_qk(*args.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Nk=0), 1, "N_k must be positive"),
    (dict(Nq=0), 1, "must be positive"),
    (dict(Nk=-3), 1, "N_k must be positive"),
    (dict(k=None), 1, "k is NULL"),
    (dict(sk=bnd.fa_strides(0, 0, 1 << 20), Nk=1024), 2, "2 GiB"),
    (dict(bmask=A, mb=64), 1, "mask_block"),
    (dict(bmask=A, Nk=300000), 2, "block mask"),
    (dict(p=1.5), 1, "dropout_p"),
])
def test_fwd_qk_rejects_bad_arguments(kw, status, msg):
    assert _fwd_qk(**kw) == status
    assert msg in fa.fa_last_error()


def test_short_python_names():
    # fa.fwd / fa.bwd are the allocating calls under their short names
    assert fa.fwd is fa.forward and fa.bwd is fa.backward


def _bwd_noalloc(**kw):
    lib = fa.load_library()
    args = dict(dtype=0, q=A, sq=S, k=A, sk=S, v=A, sv=S, o=A, so=S, do=A, sdo=S, lse=A,
                dq=A, sdq=S, dk=A, sdk=S, dv=A, sdv=S, B=1, H=1, N=1024, d=64, scale=0.125,
                causal=0, seqlens=None, bmask=None, mb=128, stream=None)
    args.update(kw)
    return lib.fa_bwd_noalloc(*args.values())


@pytest.mark.parametrize("kw,status,msg", [
    # 64 x 65537 query rows: one more than its scratch array holds
    (dict(H=64, N=65537, sq=bnd.fa_strides(0, 65537 * 64, 64)), 2, "exceed"),
    (dict(B=2, H=32, N=65537, sq=bnd.fa_strides(0, 65537 * 64, 64)), 2, "exceed"),
    (dict(dq=None), 1, "dq is NULL"),
    (dict(lse=None), 1, "lse is NULL"),
    (dict(d=96), 2, "head dimension"),
    (dict(scale=-1.0), 1, "scale"),
])
def test_bwd_noalloc_rejects_bad_arguments(kw, status, msg):
    assert _bwd_noalloc(**kw) == status
    assert msg in fa.fa_last_error()
