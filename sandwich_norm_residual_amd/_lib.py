"""ctypes view of libsnr.so (the C ABI declared in include/snr.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind these symbols. If the library has not been built this module
raises; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libsnr.so")

SNR_F32 = 0
SNR_BF16 = 1
SNR_F16 = 2

SNR_OK = 0
SNR_ERR_NULL = 1
SNR_ERR_SHAPE = 2
SNR_ERR_DTYPE = 3
SNR_ERR_EPS = 4
SNR_ERR_ALIAS = 5
SNR_ERR_ALIGN = 6
SNR_ERR_WORKSPACE = 7
SNR_ERR_HIP = 8
SNR_ERR_DEVICE = 9
SNR_ERR_CAPTURE = 10

SHAPE_AUTO = 0
SHAPE_ROWTILE = 1
SHAPE_SPLIT = 2
SHAPE_MULTIPASS = 3
SHAPE_PERSIST = 4

MAX_SEGMENTS = 8


class Segment(ctypes.Structure):
    """snr_segment: one RMSNorm problem of a rmsnorm_fwd_multi call."""
    _fields_ = [("x", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("eps", ctypes.c_float)]

# Every function include/snr.h declares, with its ctypes signature.
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_f = ctypes.c_float
_int = ctypes.c_int
SIGNATURES = {
    "rmsnorm_fwd": (_int, [_vp, _vp, _f, _i64, _i64, _int, _vp, _vp]),
    "sandwich_tail": (_int, [_vp, _vp, _vp, _f, _vp, _f, _vp, _vp, _i64,
                             _i64, _vp]),
    "sandwich_tail_noalloc": (_int, [_vp, _vp, _vp, _f, _vp, _f, _vp, _vp,
                                     _i64, _i64, _vp]),
    "sandwich_tail_typed": (_int, [_vp, _vp, _vp, _f, _vp, _f, _vp, _vp,
                                   _i64, _i64, _int, _vp]),
    "sandwich_tail_inplace": (_int, [_vp, _vp, _vp, _f, _vp, _f, _vp, _i64,
                                     _i64, _int, _vp]),
    "norm_then_add": (_int, [_vp, _vp, _vp, _f, _vp, _vp, _i64, _i64, _int,
                             _vp]),
    "add_then_norm": (_int, [_vp, _vp, _vp, _f, _vp, _vp, _i64, _i64, _int,
                             _vp]),
    "rmsnorm_q8_1": (_int, [_vp, _vp, _f, _i64, _i64, _int, _vp, _vp]),
    "rmsnorm_fwd_multi": (_int, [ctypes.POINTER(Segment), _int, _i64, _int,
                                 _vp]),
    "snr_strerror": (ctypes.c_char_p, [_int]),
    "snr_last_hip_error": (_int, []),
    "snr_force_shape": (_int, [_int, _int, _int]),
    "snr_force_grid": (_int, [_i64]),
    "snr_last_shape": (_int, [ctypes.c_char_p, _int]),
    "snr_split_timeouts": (_int, [_vp, ctypes.POINTER(_i64)]),
    "snr_release_workspaces": (_int, []),
}

_LIB = None


class SnrError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        text = strerror(code)
        if code == SNR_ERR_HIP:
            text += f" (hipError_t {lib().snr_last_hip_error()})"
        super().__init__(f"{where}: {text} [code {code}]")


def lib() -> ctypes.CDLL:
    """Load libsnr.so once; raise if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(
                f"{LIBRARY} is not built; run "
                "`python -m sandwich_norm_residual_amd.build` first")
        # PyTorch first: it bundles its own HIP runtime under the same
        # soname as the one libsnr.so links against, and a process keeps
        # whichever copy it loads first. Loading ours ahead of torch's left
        # later kernel launches failing with hipErrorNoDevice (100).
        import torch  # noqa: F401
        handle = ctypes.CDLL(LIBRARY)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def strerror(code: int) -> str:
    return lib().snr_strerror(code).decode()


def check(code: int, where: str) -> None:
    if code != SNR_OK:
        raise SnrError(code, where)


def rmsnorm_fwd(x: int, gamma: int, eps: float, rows: int, n: int,
                dtype: int, y: int, stream: int) -> int:
    """Raw call with integer device addresses; returns the SNR_* code."""
    return lib().rmsnorm_fwd(x, gamma, eps, rows, n, dtype, y, stream)


def sandwich_tail(a: int, r: int, gamma_post: int, eps_post: float,
                  gamma_pre: int, eps_pre: float, h_out: int, y_out: int,
                  rows: int, n: int, stream: int) -> int:
    """Raw call with integer device addresses; returns the SNR_* code."""
    return lib().sandwich_tail(a, r, gamma_post, eps_post, gamma_pre, eps_pre,
                               h_out, y_out, rows, n, stream)


def sandwich_tail_typed(a, r, gamma_post, eps_post, gamma_pre, eps_pre,
                        h_out, y_out, rows, n, dtype, stream) -> int:
    return lib().sandwich_tail_typed(a, r, gamma_post, eps_post, gamma_pre,
                                     eps_pre, h_out, y_out, rows, n, dtype,
                                     stream)


def sandwich_tail_inplace(a, residual, gamma_post, eps_post, gamma_pre,
                          eps_pre, y_out, rows, n, dtype, stream) -> int:
    return lib().sandwich_tail_inplace(a, residual, gamma_post, eps_post,
                                       gamma_pre, eps_pre, y_out, rows, n,
                                       dtype, stream)


def norm_then_add(a, r, gamma, eps, out_scale, out, rows, n, dtype,
                  stream) -> int:
    return lib().norm_then_add(a, r, gamma, eps, out_scale, out, rows, n,
                               dtype, stream)


def add_then_norm(a, b, gamma, eps, sum_out, y_out, rows, n, dtype,
                  stream) -> int:
    return lib().add_then_norm(a, b, gamma, eps, sum_out, y_out, rows, n,
                               dtype, stream)


def rmsnorm_q8_1(x, gamma, eps, rows, n, dtype, out, stream) -> int:
    return lib().rmsnorm_q8_1(x, gamma, eps, rows, n, dtype, out, stream)


def rmsnorm_fwd_multi(segments, n, dtype, stream) -> int:
    """segments: sequence of (x, gamma, y, rows, eps) with integer device
    addresses."""
    arr = (Segment * max(len(segments), 1))(
        *[Segment(x, g, y, rows, eps) for x, g, y, rows, eps in segments])
    return lib().rmsnorm_fwd_multi(arr, len(segments), n, dtype, stream)


def force_shape(kind: int, g: int = 0, vpt: int = 0) -> None:
    check(lib().snr_force_shape(kind, g, vpt), "snr_force_shape")


def release_workspaces() -> None:
    check(lib().snr_release_workspaces(), "snr_release_workspaces")


def force_grid(max_groups: int = 0) -> None:
    check(lib().snr_force_grid(max_groups), "snr_force_grid")


def last_shape() -> str:
    buf = ctypes.create_string_buffer(64)
    check(lib().snr_last_shape(buf, 64), "snr_last_shape")
    return buf.value.decode()


def split_timeouts(stream: int) -> int:
    out = _i64(0)
    check(lib().snr_split_timeouts(stream, ctypes.byref(out)),
          "snr_split_timeouts")
    return out.value
