"""Comparison of GPU outputs with the f64 oracle.

Metrics (the pages' "relative error" is not defined further, so this is the
reading used throughout):

* plain RMSNorm: elementwise |g - o| / |o|. Where the oracle output is exactly
  zero (a zero input element or row) the GPU must return exactly zero.
  y_j = x_j * inv_rms * gamma_j is a product, so its elementwise relative error
  is the relative error of inv_rms plus a few roundings: well conditioned.
* tail h: |g - o| / (|r_j| + |p_j|), p = the oracle's post-norm term. This is
  the natural scale of the f32 addition r + p; a plain elementwise ratio is
  unbounded wherever r_j ~ -p_j, and millions of random elements make such
  cancellations certain.
* tail y: |g - o| / (|gamma_pre_j| * (|r_j| + |p_j|) / d_h).

Where a denominator is zero the GPU value must equal the oracle's exactly.
Tolerances: f32 <= 1e-5 (the dormouse report's gate against a scalar f64
definition); bf16 <= 8e-3 (about two bf16 units 2^-8: one output rounding,
plus, on the multi-pass path only, the rounding of the stored intermediate
that its last pass re-reads; elsewhere a later norm works from the f32
intermediate);
f16 <= 2e-3 (the same budget in f16 units, 4 x 2^-11). For f16 the
denominator is at least the smallest normal 2^-14: below it f16 holds values
to an absolute 2^-25, not to a relative 2^-11.
"""
from __future__ import annotations

import numpy as np

from sandwich_norm_residual_amd.inputs import bf16_bits_to_f32

TOL_F32 = 1e-5
TOL_BF16 = 8e-3
TOL_F16 = 2e-3
TOLS = {"f32": TOL_F32, "bf16": TOL_BF16, "f16": TOL_F16}


def scaled_error(got, want, scale, floor=0.0):
    """max |got - want| / max(scale, floor), with exact equality required
    where scale is zero; non-finite GPU values count as infinite error.
    `floor` is the smallest normal of the output type: below it a storage
    type keeps absolute, not relative, precision (f16 subnormals)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    scale = np.asarray(scale, np.float64)
    if not np.all(np.isfinite(got)):
        return np.inf, int(np.count_nonzero(~np.isfinite(got)))
    diff = np.abs(got - want)
    zero = scale == 0
    bad_zero = int(np.count_nonzero(diff[zero] != 0))
    err = diff[~zero] / np.maximum(scale[~zero], floor)
    worst = float(err.max()) if err.size else 0.0
    if bad_zero:
        worst = np.inf
    return worst, bad_zero


# smallest normal value of each storage type (relative error is measured
# against at least this much)
NORMAL_MIN = {"f32": 2.0 ** -126, "bf16": 2.0 ** -126, "f16": 2.0 ** -14}


def plain_error(got, want, floor=0.0):
    return scaled_error(got, want, np.abs(want), floor)[0]


def tail_errors(h_got, y_got, oracle_result, r, gamma_pre, floor=0.0):
    o = oracle_result
    scale_h = np.abs(np.asarray(r, np.float64)) + np.abs(o.p)
    scale_y = (np.abs(np.asarray(gamma_pre, np.float64))[None, :] * scale_h /
               o.d_h[:, None])
    eh = scaled_error(h_got, o.h, scale_h, floor)[0]
    ey = scaled_error(y_got, o.y, scale_y, floor)[0]
    return eh, ey


def bf16_as_f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)
