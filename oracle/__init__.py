"""Scalar f64 CPU oracle for row-wise RMSNorm and the dual-epsilon sandwich tail.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The library's
compute path (``sandwich_norm_residual_amd``) never imports it, and this
package imports nothing from the library: the two share no code. The only
module both sides use is the seeded input generator, which holds none of the
method's arithmetic.

The arithmetic lives in ``snr_oracle.c`` (plain double-precision loops, built
with ``gcc -O2 -ffp-contract=off -fno-fast-math``); this file only marshals
numpy arrays through ctypes. Every function is pinned by
``tests/test_oracle_pins.py``; none is "parity unpinned".

Definitions followed (cited by page title and section):

* ``rmsnorm``: "RMSNorm and the dual-epsilon sandwich" (Muser book ch. 12),
  section 12.1 "What it computes": y = x / sqrt(mean(x^2) + eps) * gamma.
* ``sandwich_tail``: same page, section 12.2 (sandwich order) and section
  12.4.3 (the dual-epsilon fused tail): h = r + rmsnorm(a, gamma_post,
  eps_post); y = rmsnorm(h, gamma_pre, eps_pre), with h kept in f64.
* ``norm_then_add``: Hesper "RMSNorm Layer" page, rmsNormThenAddKernel and
  rmsNormThenAddThenBroadcastScaleKernel: (rmsnorm(a) + r) * scale.
* ``add_then_norm``: same page, residualAddRmsNormKernel: s = a + b and
  rmsnorm(s), both returned, s kept in f64.
* ``rmsnorm_q8_1``: same page, "Fused RMSNorm + Q8_1 quantize": per block of
  32 normalised values, d = amax / 127 and q = round-half-even(x / d)
  clamped to int8 (a zero block gives d = 0, q = 0).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "snr_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
          "-shared", "-fPIC"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the C oracle with gcc (host only, no HIP) and return its path."""
    tmp = output + ".tmp"
    subprocess.run(["gcc", *CFLAGS, source, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, output)
    return output


_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.c_void_p)


@dataclass
class TailResult:
    h: np.ndarray     # updated residual stream, f64 [rows, n]
    y: np.ndarray     # next pre-normed input, f64 [rows, n]
    p: np.ndarray     # post-norm term gamma_post * a / d_a, f64 [rows, n]
    d_a: np.ndarray   # post-norm denominator per row, f64 [rows]
    d_h: np.ndarray   # pre-norm denominator per row, f64 [rows]


class Oracle:
    """Handle on one compiled copy of the oracle (the mutation tests load
    deliberately broken copies through the same class)."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        lib.snr_oracle_rmsnorm_f32.argtypes = [vp, vp, ctypes.c_float, _i64,
                                               _i64, vp, vp, vp]
        lib.snr_oracle_rmsnorm_bf16.argtypes = [vp, vp, ctypes.c_float, _i64,
                                                _i64, vp, vp, vp]
        lib.snr_oracle_sandwich_tail.argtypes = [vp, vp, vp, ctypes.c_float,
                                                 vp, ctypes.c_float, _i64,
                                                 _i64, vp, vp, vp, vp, vp, vp]
        lib.snr_oracle_norm_then_add.argtypes = [vp, vp, vp, ctypes.c_float,
                                                 ctypes.c_double, _i64, _i64,
                                                 vp, vp, vp]
        lib.snr_oracle_add_then_norm.argtypes = [vp, vp, vp, ctypes.c_float,
                                                 _i64, _i64, vp, vp, vp, vp]
        lib.snr_oracle_rmsnorm_q8_1.argtypes = [vp, vp, ctypes.c_float, _i64,
                                                _i64, vp, vp, vp, vp, vp]
        for f in (lib.snr_oracle_rmsnorm_f32, lib.snr_oracle_rmsnorm_bf16,
                  lib.snr_oracle_sandwich_tail, lib.snr_oracle_norm_then_add,
                  lib.snr_oracle_add_then_norm, lib.snr_oracle_rmsnorm_q8_1):
            f.restype = ctypes.c_int
        self._lib = lib

    # -- plain RMSNorm ---------------------------------------------------
    def rmsnorm(self, x: np.ndarray, gamma: np.ndarray, eps: float,
                return_rms: bool = False):
        """x: [rows, n] float32, or uint16 holding bf16 bit patterns.
        gamma: [n] of the same storage type. Returns f64 y (and rms)."""
        x = np.ascontiguousarray(x)
        gamma = np.ascontiguousarray(gamma)
        if x.ndim != 2 or gamma.shape != (x.shape[1],):
            raise ValueError("x must be [rows, n] and gamma [n]")
        if x.dtype != gamma.dtype:
            raise ValueError("x and gamma must share a storage type")
        rows, n = x.shape
        y = np.empty((rows, n), np.float64)
        rms = np.empty(rows, np.float64)
        work = np.empty(2 * max(n, 1), np.float64)
        if x.dtype == np.float32:
            fn = self._lib.snr_oracle_rmsnorm_f32
        elif x.dtype == np.uint16:
            fn = self._lib.snr_oracle_rmsnorm_bf16
        else:
            raise ValueError(f"unsupported storage type {x.dtype}")
        rc = fn(_ptr(x), _ptr(gamma), float(eps), rows, n, _ptr(y),
                _ptr(rms), _ptr(work))
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (code {rc})")
        return (y, rms) if return_rms else y

    # -- fused dual-epsilon tail ----------------------------------------
    def sandwich_tail(self, a: np.ndarray, r: np.ndarray,
                      gamma_post: np.ndarray, eps_post: float,
                      gamma_pre: np.ndarray, eps_pre: float) -> TailResult:
        """All inputs float32; a, r: [rows, n]; gammas: [n]."""
        arrs = [np.ascontiguousarray(v, dtype=np.float32)
                for v in (a, r, gamma_post, gamma_pre)]
        a, r, gamma_post, gamma_pre = arrs
        if a.ndim != 2 or r.shape != a.shape:
            raise ValueError("a and r must both be [rows, n]")
        rows, n = a.shape
        if gamma_post.shape != (n,) or gamma_pre.shape != (n,):
            raise ValueError("gammas must be [n]")
        h = np.empty((rows, n), np.float64)
        y = np.empty((rows, n), np.float64)
        p = np.empty((rows, n), np.float64)
        d_a = np.empty(rows, np.float64)
        d_h = np.empty(rows, np.float64)
        work = np.empty(4 * max(n, 1), np.float64)
        rc = self._lib.snr_oracle_sandwich_tail(
            _ptr(a), _ptr(r), _ptr(gamma_post), float(eps_post),
            _ptr(gamma_pre), float(eps_pre), rows, n, _ptr(h), _ptr(y),
            _ptr(p), _ptr(d_a), _ptr(d_h), _ptr(work))
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (code {rc})")
        return TailResult(h, y, p, d_a, d_h)


    # -- the tail's two halves ------------------------------------------
    def norm_then_add(self, a: np.ndarray, r: np.ndarray, gamma: np.ndarray,
                      eps: float, scale: float | None = None):
        """(a / sqrt(mean(a^2) + eps) * gamma + r) * scale, f64; float32
        inputs. Returns (out, d) with d the per-row denominator."""
        a, r, gamma = (np.ascontiguousarray(v, dtype=np.float32)
                       for v in (a, r, gamma))
        if a.ndim != 2 or r.shape != a.shape or gamma.shape != (a.shape[1],):
            raise ValueError("a, r must be [rows, n] and gamma [n]")
        rows, n = a.shape
        out = np.empty((rows, n), np.float64)
        d = np.empty(rows, np.float64)
        work = np.empty(2 * max(n, 1), np.float64)
        rc = self._lib.snr_oracle_norm_then_add(
            _ptr(a), _ptr(r), _ptr(gamma), float(eps),
            1.0 if scale is None else float(scale), rows, n, _ptr(out),
            _ptr(d), _ptr(work))
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (code {rc})")
        return out, d

    def add_then_norm(self, a: np.ndarray, b: np.ndarray, gamma: np.ndarray,
                      eps: float):
        """s = a + b; y = s / sqrt(mean(s^2) + eps) * gamma, f64; float32
        inputs. Returns (s, y, d)."""
        a, b, gamma = (np.ascontiguousarray(v, dtype=np.float32)
                       for v in (a, b, gamma))
        if a.ndim != 2 or b.shape != a.shape or gamma.shape != (a.shape[1],):
            raise ValueError("a, b must be [rows, n] and gamma [n]")
        rows, n = a.shape
        s = np.empty((rows, n), np.float64)
        y = np.empty((rows, n), np.float64)
        d = np.empty(rows, np.float64)
        work = np.empty(2 * max(n, 1), np.float64)
        rc = self._lib.snr_oracle_add_then_norm(
            _ptr(a), _ptr(b), _ptr(gamma), float(eps), rows, n, _ptr(s),
            _ptr(y), _ptr(d), _ptr(work))
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (code {rc})")
        return s, y, d


    # -- RMSNorm followed by Q8_1 quantisation ---------------------------
    def rmsnorm_q8_1(self, x: np.ndarray, gamma: np.ndarray, eps: float):
        """float32 x [rows, n] (n a multiple of 32), gamma [n]. Returns
        (y, d, t, q): normalised rows (f64), block scales d = amax/127 (f64,
        [rows, n/32]), t = y/d (f64; 0 in zero blocks) and the int8 codes
        round-half-even(t) clamped to [-128, 127]."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        gamma = np.ascontiguousarray(gamma, dtype=np.float32)
        if x.ndim != 2 or gamma.shape != (x.shape[1],):
            raise ValueError("x must be [rows, n] and gamma [n]")
        rows, n = x.shape
        y = np.empty((rows, n), np.float64)
        d = np.empty((rows, max(n // 32, 0)), np.float64)
        t = np.empty((rows, n), np.float64)
        q = np.empty((rows, n), np.int8)
        work = np.empty(2 * max(n, 1), np.float64)
        rc = self._lib.snr_oracle_rmsnorm_q8_1(
            _ptr(x), _ptr(gamma), float(eps), rows, n, _ptr(y), _ptr(d),
            _ptr(t), _ptr(q), _ptr(work))
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (code {rc})")
        return y, d, t, q


_DEFAULT: Oracle | None = None


def load(rebuild: bool = False) -> Oracle:
    """Return the oracle built from ``snr_oracle.c``, compiling it first if the
    library is missing or older than its source."""
    global _DEFAULT
    stale = (not os.path.exists(LIBRARY) or
             os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE))
    if rebuild or stale:
        build()
        _DEFAULT = None
    if _DEFAULT is None:
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT
