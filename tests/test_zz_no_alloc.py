"""sandwich_tail_noalloc, the entry point for callers that cannot allocate
device memory, against sandwich_tail through the C ABI: row tiles, the
split-row kernels and the multi-pass kernels (the two that use the static
scratch array), each as two calls in a row with the second smaller, outputs
bit for bit equal to sandwich_tail's and within the f32 gate of the
oracle."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import _lib  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import check_tail, dev, host_f64, say  # noqa: E402

pytestmark = pytest.mark.gpu


def _run(fn, inp):
    a, r = dev(inp["a"], "f32"), dev(inp["r"], "f32")
    gp, gq = dev(inp["gamma_post"], "f32"), dev(inp["gamma_pre"], "f32")
    h = torch.full_like(a, float("nan"))
    y = torch.full_like(a, float("nan"))
    rows, n = inp["a"].shape
    rc = fn(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(r.data_ptr()),
            ctypes.c_void_p(gp.data_ptr()), ctypes.c_float(inp["eps_post"]),
            ctypes.c_void_p(gq.data_ptr()), ctypes.c_float(inp["eps_pre"]),
            ctypes.c_void_p(h.data_ptr()), ctypes.c_void_p(y.data_ptr()),
            ctypes.c_int64(rows), ctypes.c_int64(n),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == _lib.SNR_OK, _lib.strerror(rc)
    torch.cuda.synchronize()
    return h, y


@pytest.mark.parametrize("kind,sizes", [
    ("auto", [(64, 6656), (8, 6657)]),                  # row tiles
    ("auto", [(24, 81923), (5, 70001)]),                # split-row kernels
    ("multipass", [(6, 3 * 16384 + 3), (3, 20001)]),    # multi-pass kernels
])
def test_noalloc_matches_sandwich_tail(oracle, kind, sizes):
    L = _lib.lib()
    for i, (rows, n) in enumerate(sizes):
        say(f"noalloc {kind} call {i}: rows={rows} n={n}")
        inp = gen.random_tail(rows, n, 7100 + 10 * i + n % 97)
        with snr.forced_shape(kind):
            h0, y0 = _run(L.sandwich_tail, inp)
            want = snr.last_shape()
            h1, y1 = _run(L.sandwich_tail_noalloc, inp)
            got = snr.last_shape()
        assert got == want, (got, want)
        if kind == "multipass":
            assert got.startswith("multipass:"), got
        elif n > 65536:
            assert got.startswith("split:"), got
        assert torch.equal(h0, h1) and torch.equal(y0, y1), (kind, rows, n)
        check_tail(oracle, inp, host_f64(h1), host_f64(y1),
                   f"noalloc-{kind}-{rows}x{n}")
