"""The Python binding's own checks: tensors that cannot cross the C ABI
(host memory, mixed dtypes, strided views, wrong shapes) raise ValueError
before any call, and the stream handle passed down is the current stream."""
import pytest
import torch

import sandwich_norm_residual_amd as snr

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _tail_args(n=256, rows=4, dtype=torch.float32):
    a = torch.randn(rows, n, device=DEV).to(dtype)
    r = torch.randn(rows, n, device=DEV).to(dtype)
    g = torch.ones(n, device=DEV).to(dtype)
    return a, r, g


@pytest.mark.parametrize("bad", ["host_a", "host_gamma", "dtype_r",
                                 "strided_r", "gamma_shape", "h_shape",
                                 "y_dtype", "float64"])
def test_tail_rejects(bad):
    a, r, g = _tail_args()
    kw = {}
    if bad == "host_a":
        a = a.cpu()
    elif bad == "host_gamma":
        g = g.cpu()
    elif bad == "dtype_r":
        r = r.to(torch.bfloat16)
    elif bad == "strided_r":
        r = torch.randn(a.shape[1], a.shape[0], device=DEV).t()
    elif bad == "gamma_shape":
        g = torch.ones(a.shape[1] + 1, device=DEV)
    elif bad == "h_shape":
        kw["h_out"] = torch.empty(a.shape[0] + 1, a.shape[1], device=DEV)
    elif bad == "y_dtype":
        kw["y_out"] = torch.empty_like(a, dtype=torch.float16)
    else:
        a, r, g = (t.double() for t in (a, r, g))
    with pytest.raises(ValueError):
        snr.sandwich_tail(a, r, g, 1e-8, g, 1e-5, **kw)


def test_other_entry_points_reject_mismatches():
    a, r, g = _tail_args()
    with pytest.raises(ValueError):
        snr.rmsnorm_fwd(a, g.to(torch.bfloat16), 1e-5)
    with pytest.raises(ValueError):
        snr.rmsnorm_fwd(a, g, 1e-5, out=torch.empty(3, device=DEV))
    with pytest.raises(ValueError):
        snr.norm_then_add(a, r, g, 1e-8,
                          out_scale=torch.ones(1, device=DEV,
                                               dtype=torch.float16))
    with pytest.raises(ValueError):
        snr.add_then_norm(a, r[:, :128].contiguous(), g, 1e-5)
    with pytest.raises(ValueError):
        snr.sandwich_tail_inplace(a, r.t(), g, 1e-8, g, 1e-5)
    with pytest.raises(ValueError):
        snr.rmsnorm_fwd_multi([(a, g, 1e-5), (a.to(torch.bfloat16), g, 1e-5)])
    with pytest.raises(ValueError):
        snr.rmsnorm_q8_1(a, g, 1e-5, out=torch.empty(4, 8, 36, device=DEV))


def test_stream_handle_is_the_current_stream():
    from sandwich_norm_residual_amd import _stream
    dev = torch.device(DEV)
    assert _stream(dev) == torch.cuda.current_stream(dev).cuda_stream
    s = torch.cuda.Stream()   # default priority
    with torch.cuda.stream(s):
        assert _stream(dev) == s.cuda_stream
        a, r, g = _tail_args(n=6656, rows=8)
        h, y = snr.sandwich_tail(a, r, g, 1e-8, g, 1e-5)
    s.synchronize()
    h2, y2 = snr.sandwich_tail(a, r, g, 1e-8, g, 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(h, h2) and torch.equal(y, y2)
