"""The C-ABI library loads, exports every symbol include/snr.h declares, and
rejects bad arguments with the documented codes. CPU only: every call here
fails validation before the library makes any HIP call (fake, never
dereferenced addresses), so no GPU is touched."""
import ctypes
import math
import os
import re
import subprocess

import pytest

from sandwich_norm_residual_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "snr.h")


def _header_text():
    with open(HEADER) as fh:
        return fh.read()


def declared_functions():
    return set(re.findall(r"^SNR_API\s+[\w\s\*]*?\b(\w+)\s*\(", _header_text(), re.M))


def header_enum(name):
    m = re.search(rf"\b{name}\s*=\s*(\d+)", _header_text())
    assert m, name
    return int(m.group(1))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_header_declares_the_two_entry_points():
    fns = declared_functions()
    assert {"rmsnorm_fwd", "sandwich_tail"} <= fns
    assert fns == set(_lib.SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIBRARY],
                         capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = declared_functions() - exported
    assert not missing, missing
    for name in declared_functions():
        assert getattr(L, name) is not None


def test_error_codes_match_header():
    for name in ["SNR_OK", "SNR_ERR_NULL", "SNR_ERR_SHAPE", "SNR_ERR_DTYPE",
                 "SNR_ERR_EPS", "SNR_ERR_ALIAS", "SNR_ERR_ALIGN",
                 "SNR_ERR_WORKSPACE", "SNR_ERR_HIP", "SNR_ERR_DEVICE",
                 "SNR_ERR_CAPTURE",
                 "SNR_F32", "SNR_BF16", "SNR_F16"]:
        assert header_enum(name) == getattr(_lib, name), name
    assert header_enum("SNR_SHAPE_ROWTILE") == _lib.SHAPE_ROWTILE
    assert header_enum("SNR_SHAPE_SPLIT") == _lib.SHAPE_SPLIT
    assert header_enum("SNR_SHAPE_MULTIPASS") == _lib.SHAPE_MULTIPASS


def test_strerror_covers_every_code(L):
    seen = set()
    for code in range(11):
        text = _lib.strerror(code)
        assert text and text != "unknown error code", code
        seen.add(text)
    assert len(seen) == 11
    assert _lib.strerror(12345) == "unknown error code"


BASE = 1 << 32          # fake device addresses, 16-byte aligned, never used
GAM = BASE + (1 << 28)
OUT = BASE + (1 << 29)


def plain(x=BASE, g=GAM, eps=1e-5, rows=4, n=64, dtype=_lib.SNR_F32, y=OUT):
    return _lib.rmsnorm_fwd(x, g, eps, rows, n, dtype, y, 0)


def tail(a=BASE, r=BASE + (1 << 26), gp=GAM, ep=1e-8, gq=GAM + (1 << 20),
         eq=1e-5, h=OUT, y=OUT + (1 << 26), rows=4, n=64):
    return _lib.sandwich_tail(a, r, gp, ep, gq, eq, h, y, rows, n, 0)


def test_plain_argument_errors(L):
    assert plain(x=0) == _lib.SNR_ERR_NULL
    assert plain(g=0) == _lib.SNR_ERR_NULL
    assert plain(y=0) == _lib.SNR_ERR_NULL
    assert plain(n=0) == _lib.SNR_ERR_SHAPE
    assert plain(n=-3) == _lib.SNR_ERR_SHAPE
    assert plain(n=2 ** 31) == _lib.SNR_ERR_SHAPE
    assert plain(rows=-1) == _lib.SNR_ERR_SHAPE
    assert plain(rows=2 ** 62, n=2 ** 20) == _lib.SNR_ERR_SHAPE
    assert plain(dtype=3) == _lib.SNR_ERR_DTYPE
    assert plain(dtype=-1) == _lib.SNR_ERR_DTYPE
    for bad in (0.0, -1e-5, math.nan, math.inf, -math.inf):
        assert plain(eps=bad) == _lib.SNR_ERR_EPS, bad
    assert plain(x=BASE + 2) == _lib.SNR_ERR_ALIGN
    assert plain(y=OUT + 1, dtype=_lib.SNR_BF16) == _lib.SNR_ERR_ALIGN
    # y partially overlapping x, or overlapping gamma
    assert plain(y=BASE + 4) == _lib.SNR_ERR_ALIAS
    assert plain(y=GAM - 8) == _lib.SNR_ERR_ALIAS
    assert plain(x=GAM, y=GAM) == _lib.SNR_ERR_ALIAS  # in place over gamma


def test_plain_rows_zero_is_a_noop_even_with_null_pointers(L):
    assert plain(x=0, g=0, y=0, rows=0) == _lib.SNR_OK


def test_tail_argument_errors(L):
    assert tail(a=0) == _lib.SNR_ERR_NULL
    assert tail(y=0) == _lib.SNR_ERR_NULL
    assert tail(n=0) == _lib.SNR_ERR_SHAPE
    assert tail(rows=-2) == _lib.SNR_ERR_SHAPE
    assert tail(ep=0.0) == _lib.SNR_ERR_EPS
    assert tail(eq=math.nan) == _lib.SNR_ERR_EPS
    assert tail(h=OUT + 2) == _lib.SNR_ERR_ALIGN
    r = BASE + (1 << 26)
    assert tail(h=BASE) == _lib.SNR_ERR_ALIAS           # h over a
    assert tail(y=r) == _lib.SNR_ERR_ALIAS              # y over r
    assert tail(y=OUT) == _lib.SNR_ERR_ALIAS            # y over h
    assert tail(h=r + 16) == _lib.SNR_ERR_ALIAS         # h partly over r
    assert tail(y=GAM) == _lib.SNR_ERR_ALIAS            # y over a gain
    assert tail(h=GAM + (1 << 20) - 4) == _lib.SNR_ERR_ALIAS  # h over gamma_pre
    assert tail(a=0, r=0, gp=0, gq=0, h=0, y=0, rows=0) == _lib.SNR_OK


def test_force_shape_rejects_unknown_kind(L):
    assert L.snr_force_shape(7, 0, 0) == _lib.SNR_ERR_SHAPE
    for name in ("ROWTILE", "SPLIT", "MULTIPASS", "PERSIST"):
        code = header_enum(f"SNR_SHAPE_{name}")
        assert code == getattr(_lib, f"SHAPE_{name}")
        assert L.snr_force_shape(code, 128, 2) == _lib.SNR_OK
    assert L.snr_force_shape(_lib.SHAPE_AUTO, 0, 0) == _lib.SNR_OK
    buf = ctypes.create_string_buffer(8)
    assert L.snr_last_shape(None, 8) == _lib.SNR_ERR_NULL
    assert L.snr_last_shape(buf, 8) == _lib.SNR_OK


def test_force_grid_rejects_a_negative_cap(L):
    assert L.snr_force_grid(-1) == _lib.SNR_ERR_SHAPE
    assert L.snr_force_grid(3) == _lib.SNR_OK
    assert L.snr_force_grid(0) == _lib.SNR_OK


R = BASE + (1 << 26)
GQ = GAM + (1 << 20)


def test_typed_and_inplace_tail_argument_errors(L):
    f = _lib.sandwich_tail_typed
    ok = dict(a=BASE, r=R, gp=GAM, ep=1e-8, gq=GQ, eq=1e-5, h=OUT,
              y=OUT + (1 << 26), rows=4, n=64, dt=_lib.SNR_BF16)

    def call(**kw):
        k = {**ok, **kw}
        return f(k["a"], k["r"], k["gp"], k["ep"], k["gq"], k["eq"], k["h"],
                 k["y"], k["rows"], k["n"], k["dt"], 0)

    assert call(dt=9) == _lib.SNR_ERR_DTYPE
    assert call(a=BASE + 1) == _lib.SNR_ERR_ALIGN      # bf16 needs 2 bytes
    assert call(dt=_lib.SNR_F32, a=BASE + 2) == _lib.SNR_ERR_ALIGN
    assert call(y=R) == _lib.SNR_ERR_ALIAS
    assert call(h=R + 2) == _lib.SNR_ERR_ALIAS
    assert call(gp=0) == _lib.SNR_ERR_NULL
    assert call(ep=-1.0) == _lib.SNR_ERR_EPS
    assert call(rows=0, a=0, r=0, gp=0, gq=0, h=0, y=0) == _lib.SNR_OK
    g = _lib.sandwich_tail_inplace
    assert g(BASE, R, GAM, 1e-8, GQ, 1e-5, R, 4, 64, 0, 0) == \
        _lib.SNR_ERR_ALIAS                              # y over the residual
    assert g(BASE, BASE, GAM, 1e-8, GQ, 1e-5, OUT, 4, 64, 0, 0) == \
        _lib.SNR_ERR_ALIAS                              # residual over a
    assert g(BASE, R, GAM, 1e-8, GQ, 1e-5, OUT, 4, 64, 5, 0) == \
        _lib.SNR_ERR_DTYPE


def test_norm_then_add_argument_errors(L):
    f = _lib.norm_then_add
    SC = GAM + (1 << 22)
    assert f(0, R, GAM, 1e-8, None, OUT, 4, 64, 0, 0) == _lib.SNR_ERR_NULL
    assert f(BASE, R, GAM, 0.0, None, OUT, 4, 64, 0, 0) == _lib.SNR_ERR_EPS
    assert f(BASE, R, GAM, 1e-8, SC + 1, OUT, 4, 64, 0, 0) == \
        _lib.SNR_ERR_ALIGN                              # scale not f32-aligned
    assert f(BASE, R, GAM, 1e-8, None, BASE, 4, 64, 0, 0) == \
        _lib.SNR_ERR_ALIAS                              # out over a
    assert f(BASE, R, GAM, 1e-8, None, R + 4, 4, 64, 0, 0) == \
        _lib.SNR_ERR_ALIAS                              # out partly over r
    assert f(BASE, R, GAM, 1e-8, R + 8, R, 4, 64, 0, 0) == \
        _lib.SNR_ERR_ALIAS                              # scale inside out
    assert f(BASE, R, GAM, 1e-8, None, OUT, 4, 64, 3, 0) == \
        _lib.SNR_ERR_DTYPE
    assert f(0, 0, 0, 1e-8, None, 0, 0, 64, 0, 0) == _lib.SNR_OK


def test_add_then_norm_argument_errors(L):
    f = _lib.add_then_norm
    Y = OUT + (1 << 26)
    assert f(BASE, R, GAM, 1e-5, OUT, 0, 4, 64, 0, 0) == _lib.SNR_ERR_NULL
    assert f(BASE, R, GAM, math.inf, OUT, Y, 4, 64, 0, 0) == _lib.SNR_ERR_EPS
    assert f(BASE, R, GAM, 1e-5, OUT, BASE, 4, 64, 0, 0) == \
        _lib.SNR_ERR_ALIAS                              # y over a
    assert f(BASE, R, GAM, 1e-5, OUT, OUT + 8, 4, 64, 0, 0) == \
        _lib.SNR_ERR_ALIAS                              # y over the sum
    assert f(BASE, R, GAM, 1e-5, BASE + 4, Y, 4, 64, 0, 0) == \
        _lib.SNR_ERR_ALIAS                              # sum partly over a
    assert f(BASE, R, GAM, 1e-5, GAM, Y, 4, 64, 0, 0) == \
        _lib.SNR_ERR_ALIAS                              # sum over gamma
    assert f(BASE, R, GAM, 1e-5, OUT, Y, 4, 64, _lib.SNR_F16 + 1, 0) == \
        _lib.SNR_ERR_DTYPE
    assert f(0, 0, 0, 1e-5, 0, 0, 0, 64, 0, 0) == _lib.SNR_OK


def test_multi_argument_errors(L):
    Seg = _lib.Segment

    def call(segs, count=None, n=64, dt=0):
        arr = (Seg * max(len(segs), 1))(*segs)
        return L.rmsnorm_fwd_multi(arr, len(segs) if count is None else count,
                                   n, dt, 0)

    good = Seg(BASE, GAM, OUT, 4, 1e-5)
    other = Seg(R, GQ, OUT + (1 << 26), 8, 1e-5)
    assert call([good], count=0) == _lib.SNR_ERR_SHAPE
    assert call([good] * 9) == _lib.SNR_ERR_SHAPE
    assert L.rmsnorm_fwd_multi(None, 1, 64, 0, 0) == _lib.SNR_ERR_NULL
    assert call([good, Seg(0, GQ, OUT + (1 << 26), 8, 1e-5)]) == \
        _lib.SNR_ERR_NULL
    assert call([good, Seg(R, GQ, OUT + (1 << 26), 8, 0.0)]) == \
        _lib.SNR_ERR_EPS
    assert call([good, other], dt=7) == _lib.SNR_ERR_DTYPE
    assert call([good, Seg(R, GQ, OUT + 4, 8, 1e-5)]) == \
        _lib.SNR_ERR_ALIAS                          # outputs overlap
    assert call([good, Seg(OUT, GQ, OUT + (1 << 26), 8, 1e-5)]) == \
        _lib.SNR_ERR_ALIAS                          # y of one is x of another
    assert call([good, Seg(R, OUT, OUT + (1 << 26), 8, 1e-5)]) == \
        _lib.SNR_ERR_ALIAS                          # a gain inside an output
    assert call([Seg(0, 0, 0, 0, 1e-5), Seg(0, 0, 0, 0, 1e-5)]) == \
        _lib.SNR_OK                                 # nothing to do


def test_q8_1_argument_errors(L):
    f = _lib.rmsnorm_q8_1
    assert f(BASE, GAM, 1e-5, 4, 48, 0, OUT, 0) == _lib.SNR_ERR_SHAPE  # 32∤n
    assert f(BASE, GAM, 1e-5, 4, 16, 0, OUT, 0) == _lib.SNR_ERR_SHAPE
    assert f(BASE, GAM, 1e-5, 4, 64, 3, OUT, 0) == _lib.SNR_ERR_DTYPE
    assert f(BASE, GAM, 0.0, 4, 64, 0, OUT, 0) == _lib.SNR_ERR_EPS
    assert f(BASE, 0, 1e-5, 4, 64, 0, OUT, 0) == _lib.SNR_ERR_NULL
    assert f(BASE, GAM, 1e-5, 4, 64, 0, 0, 0) == _lib.SNR_ERR_NULL
    assert f(BASE, GAM, 1e-5, 4, 64, 0, OUT + 2, 0) == _lib.SNR_ERR_ALIGN
    assert f(BASE + 2, GAM, 1e-5, 4, 64, 0, OUT, 0) == _lib.SNR_ERR_ALIGN
    assert f(BASE, GAM, 1e-5, 4, 64, 0, BASE + 64, 0) == \
        _lib.SNR_ERR_ALIAS                          # records over x
    assert f(BASE, GAM, 1e-5, 4, 64, 0, GAM - 16, 0) == \
        _lib.SNR_ERR_ALIAS                          # records over gamma
    assert f(0, 0, 1e-5, 0, 64, 0, 0, 0) == _lib.SNR_OK
