"""sandwich_norm_residual_amd - row-wise RMSNorm and the fused dual-epsilon
sandwich tail on AMD Instinct MI355X (gfx950).

The compute is done by hand-written HIP kernels in ``libsnr.so`` behind a C
ABI (``include/snr.h``); this module marshals torch tensors (device memory and
the current stream) into those calls. Nothing here computes.

    y    = rmsnorm_fwd(x, gamma, eps)                       # f32 or bf16
    h, y = sandwich_tail(a, r, gamma_post, eps_post, gamma_pre, eps_pre)

Definitions ("RMSNorm and the dual-epsilon sandwich", Muser book chapter 12):
section 12.1 for RMSNorm, sections 12.2 and 12.4.3 for the tail.
"""
from __future__ import annotations

import contextlib

from . import _lib
from ._lib import SnrError

__all__ = ["rmsnorm_fwd", "sandwich_tail", "forced_shape", "last_shape",
           "split_timeouts", "SnrError"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return _lib.SNR_F32
    if t.dtype == torch.bfloat16:
        return _lib.SNR_BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _check_tensor(name, t, device, dtype, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                         f"{tuple(shape)}")


def _rows_n(t):
    if t.dim() == 0:
        raise ValueError("expected at least one dimension")
    n = t.shape[-1]
    rows = t.numel() // n if n else 0
    return rows, n


def rmsnorm_fwd(x, gamma, eps: float, out=None):
    """y = x / sqrt(mean(x^2, -1) + eps) * gamma over the last dimension.

    x: contiguous [..., n] float32 or bfloat16 GPU tensor; gamma: [n] of the
    same dtype. ``out`` may be given (same shape and dtype; ``out is x``
    computes in place). Runs on the current stream of x's device.
    """
    torch = _torch()
    _dtype_code(x)
    _check_tensor("x", x, x.device, x.dtype)
    rows, n = _rows_n(x)
    _check_tensor("gamma", gamma, x.device, x.dtype, (n,))
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_tensor("out", out, x.device, x.dtype, x.shape)
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = _lib.rmsnorm_fwd(x.data_ptr(), gamma.data_ptr(), float(eps),
                              rows, n, _dtype_code(x), out.data_ptr(), stream)
    _lib.check(rc, "rmsnorm_fwd")
    return out


def sandwich_tail(a, r, gamma_post, eps_post: float, gamma_pre,
                  eps_pre: float, h_out=None, y_out=None):
    """The fused dual-epsilon tail over the last dimension (float32):

        h = r + gamma_post * a / sqrt(mean(a^2) + eps_post)
        y = gamma_pre * h / sqrt(mean(h^2) + eps_pre)

    Returns (h, y). ``h_out is r`` updates the residual stream in place.
    """
    torch = _torch()
    dev = a.device
    f32 = torch.float32
    _check_tensor("a", a, dev, f32)
    rows, n = _rows_n(a)
    _check_tensor("r", r, dev, f32, a.shape)
    _check_tensor("gamma_post", gamma_post, dev, f32, (n,))
    _check_tensor("gamma_pre", gamma_pre, dev, f32, (n,))
    h_out = torch.empty_like(a) if h_out is None else h_out
    y_out = torch.empty_like(a) if y_out is None else y_out
    _check_tensor("h_out", h_out, dev, f32, a.shape)
    _check_tensor("y_out", y_out, dev, f32, a.shape)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = _lib.sandwich_tail(a.data_ptr(), r.data_ptr(),
                                gamma_post.data_ptr(), float(eps_post),
                                gamma_pre.data_ptr(), float(eps_pre),
                                h_out.data_ptr(), y_out.data_ptr(), rows, n,
                                stream)
    _lib.check(rc, "sandwich_tail")
    return h_out, y_out


@contextlib.contextmanager
def forced_shape(kind: str, g: int = 0, vpt: int = 0):
    """Force a dispatch shape ("rowtile", "split" or "multipass") for calls
    made on this thread inside the block (diagnostics and tests)."""
    code = {"auto": _lib.SHAPE_AUTO, "rowtile": _lib.SHAPE_ROWTILE,
            "split": _lib.SHAPE_SPLIT, "multipass": _lib.SHAPE_MULTIPASS}[kind]
    _lib.force_shape(code, g, vpt)
    try:
        yield
    finally:
        _lib.force_shape(_lib.SHAPE_AUTO)


def last_shape() -> str:
    """"kind:g:vpt:width[:chunks]" of this thread's most recent launch
    (width = elements per 128-bit vector)."""
    return _lib.last_shape()


def split_timeouts(stream=None) -> int:
    """Bounded-wait overruns recorded by split-row kernels on a stream (0 when
    every wait completed). Synchronises the stream."""
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return _lib.split_timeouts(s.cuda_stream)
