"""sandwich_norm_residual_amd - row-wise RMSNorm and the fused dual-epsilon
sandwich tail on AMD Instinct MI355X (gfx950).

The compute is done by hand-written HIP kernels in ``libsnr.so`` behind a C
ABI (``include/snr.h``); this module marshals torch tensors (device memory and
the current stream) into those calls. Nothing here computes.

    y    = rmsnorm_fwd(x, gamma, eps)              # f32, bf16 or f16
    h, y = sandwich_tail(a, r, gamma_post, eps_post, gamma_pre, eps_pre)
    y    = sandwich_tail_inplace(a, residual, gamma_post, eps_post,
                                 gamma_pre, eps_pre)   # residual updated
    out  = norm_then_add(a, r, gamma, eps, out_scale=None)
    s, y = add_then_norm(a, b, gamma, eps)
    yq, yk = rmsnorm_fwd_multi([(q, gamma_q, eps), (k, gamma_k, eps)])
    blocks = rmsnorm_q8_1(x, gamma, eps)   # uint8 [..., n / 32, 36]

Definitions: "RMSNorm and the dual-epsilon sandwich" (Muser book chapter
12), section 12.1 for RMSNorm and sections 12.2 and 12.4.3 for the tail;
Hesper's "RMSNorm Layer" page for norm_then_add (rmsNormThenAdd kernels)
and add_then_norm (residualAddRmsNormKernel), and its "Fused RMSNorm + Q8_1
quantize" section for rmsnorm_q8_1.
"""
from __future__ import annotations

import contextlib

from . import _lib
from ._lib import SnrError

__all__ = ["rmsnorm_fwd", "rmsnorm_fwd_multi", "sandwich_tail",
           "sandwich_tail_inplace", "norm_then_add", "add_then_norm",
           "rmsnorm_q8_1", "q8_1_fields",
           "forced_shape", "forced_grid", "last_shape", "split_timeouts",
           "release_workspaces", "SnrError"]


def _torch():
    import torch
    return torch


def _on(dev):
    """A context that makes `dev` current only when it is not already (the
    switch costs a few microseconds per call)."""
    torch = _torch()
    if dev.index is None or dev.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(dev)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return _lib.SNR_F32
    if t.dtype == torch.bfloat16:
        return _lib.SNR_BF16
    if t.dtype == torch.float16:
        return _lib.SNR_F16
    raise ValueError(f"unsupported dtype {t.dtype} "
                     "(float32, bfloat16 or float16)")


def _check_tensor(name, t, device, dtype, shape=None):
    """Raise ValueError unless t is a contiguous tensor on `device` (a GPU)
    of `dtype` and, when given, `shape`. One combined test on the common
    path: each tensor attribute read costs about 0.1 us in Python."""
    if (t.dtype is dtype and t.device == device and t.is_contiguous()
            and (shape is None or t.shape == shape)):
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                     f"{tuple(shape)}")


def _lead(name, t):
    """Check the tensor that fixes a call's device and dtype; return its
    dtype code."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    code = _dtype_code(t)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return code


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
    rows, n, code = _rows_inputs([("x", x)], [("gamma", gamma)], x)
    if out is None:
        out = torch.empty_like(x)
    else:
        _outputs([("out", out)], x)
    with _on(x.device):
        rc = _lib.rmsnorm_fwd(x.data_ptr(), gamma.data_ptr(), float(eps),
                              rows, n, code, out.data_ptr(), _stream(x.device))
    _lib.check(rc, "rmsnorm_fwd")
    return out


def rmsnorm_fwd_multi(problems, outs=None):
    """Several RMSNorms of one row width and dtype in one launch.

    problems: sequence of (x, gamma, eps) with x [..., n] and gamma [n], all
    on one device; outs: optional matching outputs (``out is x`` computes in
    place). Returns the list of outputs. Up to 8 problems per call."""
    torch = _torch()
    if not problems:
        return []
    if len(problems) > _lib.MAX_SEGMENTS:
        raise ValueError(f"at most {_lib.MAX_SEGMENTS} problems per call")
    x0 = problems[0][0]
    code = _lead("x[0]", x0)
    n = x0.shape[-1]
    outs = list(outs) if outs is not None else [None] * len(problems)
    segs = []
    for i, (x, g, eps) in enumerate(problems):
        _check_tensor(f"x[{i}]", x, x0.device, x0.dtype)
        rows, nn = _rows_n(x)
        if nn != n:
            raise ValueError("all problems must share the row width")
        _check_tensor(f"gamma[{i}]", g, x0.device, x0.dtype, (n,))
        if outs[i] is None:
            outs[i] = torch.empty_like(x)
        _check_tensor(f"out[{i}]", outs[i], x0.device, x0.dtype, x.shape)
        segs.append((x.data_ptr(), g.data_ptr(), outs[i].data_ptr(), rows,
                     float(eps)))
    with _on(x0.device):
        rc = _lib.rmsnorm_fwd_multi(segs, n, code, _stream(x0.device))
    _lib.check(rc, "rmsnorm_fwd_multi")
    return outs


def _stream(dev):
    """The raw handle of `dev`'s current stream. torch's own C accessor is
    used where it exists (about 0.2 us against 1.8 us for building the
    Stream object)."""
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None and dev.index is not None:
        return raw(dev.index)
    return torch.cuda.current_stream(dev).cuda_stream


def _rows_inputs(names_tensors, gains, like):
    """Check [..., n] inputs of like's dtype, device and shape, and [n]
    gains. Returns (rows, n, dtype code); `like` itself is checked as the
    first of names_tensors."""
    code = _lead(names_tensors[0][0], like)
    dev, dt, shape = like.device, like.dtype, like.shape
    rows, n = _rows_n(like)
    for name, t in names_tensors[1:]:
        _check_tensor(name, t, dev, dt, shape)
    for name, g in gains:
        _check_tensor(name, g, dev, dt, (n,))
    return rows, n, code


def _outputs(names_tensors, like):
    """Check caller-given outputs against like's dtype, device and shape."""
    dev, dt, shape = like.device, like.dtype, like.shape
    for name, t in names_tensors:
        _check_tensor(name, t, dev, dt, shape)


def sandwich_tail(a, r, gamma_post, eps_post: float, gamma_pre,
                  eps_pre: float, h_out=None, y_out=None):
    """The fused dual-epsilon tail over the last dimension:

        h = r + gamma_post * a / sqrt(mean(a^2) + eps_post)
        y = gamma_pre * h / sqrt(mean(h^2) + eps_pre)

    Tensors share one dtype (float32, bfloat16 or float16). Returns (h, y).
    ``h_out is r`` updates the residual stream in place.
    """
    torch = _torch()
    rows, n, code = _rows_inputs([("a", a), ("r", r)],
                                 [("gamma_post", gamma_post),
                                  ("gamma_pre", gamma_pre)], a)
    if h_out is None:
        h_out = torch.empty_like(a)
    else:
        _outputs([("h_out", h_out)], a)
    if y_out is None:
        y_out = torch.empty_like(a)
    else:
        _outputs([("y_out", y_out)], a)
    with _on(a.device):
        if code == _lib.SNR_F32:
            rc = _lib.sandwich_tail(a.data_ptr(), r.data_ptr(),
                                    gamma_post.data_ptr(), float(eps_post),
                                    gamma_pre.data_ptr(), float(eps_pre),
                                    h_out.data_ptr(), y_out.data_ptr(), rows,
                                    n, _stream(a.device))
        else:
            rc = _lib.sandwich_tail_typed(
                a.data_ptr(), r.data_ptr(), gamma_post.data_ptr(),
                float(eps_post), gamma_pre.data_ptr(), float(eps_pre),
                h_out.data_ptr(), y_out.data_ptr(), rows, n, code,
                _stream(a.device))
    _lib.check(rc, "sandwich_tail")
    return h_out, y_out


def sandwich_tail_inplace(a, residual, gamma_post, eps_post: float,
                          gamma_pre, eps_pre: float, y_out=None):
    """The tail with the residual stream updated in place:
    residual += post-norm(a); returns y, the pre-norm of the updated
    residual."""
    torch = _torch()
    rows, n, code = _rows_inputs([("a", a), ("residual", residual)],
                                 [("gamma_post", gamma_post),
                                  ("gamma_pre", gamma_pre)], a)
    if y_out is None:
        y_out = torch.empty_like(a)
    else:
        _outputs([("y_out", y_out)], a)
    with _on(a.device):
        rc = _lib.sandwich_tail_inplace(
            a.data_ptr(), residual.data_ptr(), gamma_post.data_ptr(),
            float(eps_post), gamma_pre.data_ptr(), float(eps_pre),
            y_out.data_ptr(), rows, n, code, _stream(a.device))
    _lib.check(rc, "sandwich_tail_inplace")
    return y_out


def norm_then_add(a, r, gamma, eps: float, out_scale=None, out=None):
    """out = (a / sqrt(mean(a^2) + eps) * gamma + r) * out_scale[0].

    out_scale: None, or a one-element float32 GPU tensor (read on the GPU).
    ``out is r`` updates the residual in place."""
    torch = _torch()
    rows, n, code = _rows_inputs([("a", a), ("r", r)], [("gamma", gamma)], a)
    if out is None:
        out = torch.empty_like(a)
    else:
        _outputs([("out", out)], a)
    scale_ptr = None
    if out_scale is not None:
        _check_tensor("out_scale", out_scale, a.device, torch.float32)
        if out_scale.numel() < 1:
            raise ValueError("out_scale must hold one element")
        scale_ptr = out_scale.data_ptr()
    with _on(a.device):
        rc = _lib.norm_then_add(a.data_ptr(), r.data_ptr(), gamma.data_ptr(),
                                float(eps), scale_ptr, out.data_ptr(), rows,
                                n, code, _stream(a.device))
    _lib.check(rc, "norm_then_add")
    return out


def add_then_norm(a, b, gamma, eps: float, sum_out=None, y_out=None):
    """s = a + b; y = s / sqrt(mean(s^2) + eps) * gamma. Returns (s, y).
    ``sum_out`` may be ``a`` or ``b`` (accumulate in place)."""
    torch = _torch()
    rows, n, code = _rows_inputs([("a", a), ("b", b)], [("gamma", gamma)], a)
    if sum_out is None:
        sum_out = torch.empty_like(a)
    else:
        _outputs([("sum_out", sum_out)], a)
    if y_out is None:
        y_out = torch.empty_like(a)
    else:
        _outputs([("y_out", y_out)], a)
    with _on(a.device):
        rc = _lib.add_then_norm(a.data_ptr(), b.data_ptr(), gamma.data_ptr(),
                                float(eps), sum_out.data_ptr(),
                                y_out.data_ptr(), rows, n, code,
                                _stream(a.device))
    _lib.check(rc, "add_then_norm")
    return sum_out, y_out


def rmsnorm_q8_1(x, gamma, eps: float, out=None):
    """RMSNorm of each row of x, encoded as Q8_1 records: per 32 values a
    36-byte record {f16 d, f16 s = 0, int8 q[32]} with d = amax / 127 and
    q = round-half-even(v / d) clamped to [-128, 127].

    x: contiguous [..., n] GPU tensor (float32, bfloat16 or float16) with n a
    multiple of 32; gamma: [n] of the same dtype. Returns (or fills ``out``)
    a uint8 tensor [..., n / 32, 36]."""
    torch = _torch()
    rows, n, code = _rows_inputs([("x", x)], [("gamma", gamma)], x)
    if n % 32:
        raise ValueError(f"rmsnorm_q8_1 needs n a multiple of 32, got {n}")
    shape = tuple(x.shape[:-1]) + (n // 32, 36)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=x.device)
    else:
        _check_tensor("out", out, x.device, torch.uint8, shape)
    with _on(x.device):
        rc = _lib.rmsnorm_q8_1(x.data_ptr(), gamma.data_ptr(), float(eps),
                               rows, n, code, out.data_ptr(),
                               _stream(x.device))
    _lib.check(rc, "rmsnorm_q8_1")
    return out


def q8_1_fields(blocks):
    """Split Q8_1 records (uint8 [..., 36], any device) into their fields:
    (d as float16 [...], s as float16 [...], q as int8 [..., 32]). A view
    of the bytes only; nothing is computed."""
    b = blocks.contiguous()
    d = b[..., 0:2].contiguous().view(_torch().float16)[..., 0]
    s = b[..., 2:4].contiguous().view(_torch().float16)[..., 0]
    q = b[..., 4:36].contiguous().view(_torch().int8)
    return d, s, q


@contextlib.contextmanager
def forced_shape(kind: str, g: int = 0, vpt: int = 0):
    """Force a dispatch shape ("rowtile", "persist", "split" or "multipass")
    for calls made on this thread inside the block (diagnostics and tests)."""
    code = {"auto": _lib.SHAPE_AUTO, "rowtile": _lib.SHAPE_ROWTILE,
            "split": _lib.SHAPE_SPLIT, "multipass": _lib.SHAPE_MULTIPASS,
            "persist": _lib.SHAPE_PERSIST}[kind]
    _lib.force_shape(code, g, vpt)
    try:
        yield
    finally:
        _lib.force_shape(_lib.SHAPE_AUTO)


def release_workspaces() -> None:
    """Free the current device's wide-row workspaces (after their last
    uses); the next wide-row call allocates again. Workspaces recorded into a
    HIP graph are kept."""
    _lib.release_workspaces()


@contextlib.contextmanager
def forced_grid(max_groups: int):
    """Cap the rows in flight (workgroups of the persistent tiles, and per
    chunk of the split-row kernels) for calls made on this thread inside the
    block, so each workgroup walks more rows (diagnostics and tests)."""
    _lib.force_grid(max_groups)
    try:
        yield
    finally:
        _lib.force_grid(0)


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
