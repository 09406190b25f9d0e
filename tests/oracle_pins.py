"""Pins that tie the f64 oracle to something other than itself.

Each ``pin_*`` function takes a loaded oracle handle and raises
AssertionError (or any exception) if the oracle disagrees with:

* the values the Muser book prints for its worked example (section 12.3 of
  "RMSNorm and the dual-epsilon sandwich", Figure 12.1; golden file
  ``golden/rmsnorm_worked_example.txt``);
* closed forms that follow from the definition in section 12.1 (constant rows,
  n = 1 and n = 2 rows, zero rows, epsilon-dominated rows);
* invariants (mean of y^2 with unit gain, scale invariance under powers of two,
  row independence);
* library routines: ``torch.nn.functional.rms_norm`` in f64 (one of the public
  references the dormouse report uses) and, on exactly mean-centred rows,
  ``torch.nn.functional.layer_norm`` (section 12.2: mean(x^2) = var + mean^2,
  so the two coincide when the mean is zero);
* exact rational arithmetic (Python ``decimal`` at 50 digits) on tiny inputs,
  for the plain norm in f32 and bf16 storage and for the fused tail, with rows
  sized so that both epsilons of the tail matter.

The functions are plain callables so that ``test_oracle_mutants.py`` can run
the same pins against deliberately broken copies of the oracle.
"""
from __future__ import annotations

import math
import os
from decimal import Decimal, getcontext

import numpy as np

from sandwich_norm_residual_amd.inputs import (bf16_bits_to_f32,
                                                f32_to_bf16_bits, rng_for)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32 = np.float32


def _f(v) -> float:
    """The exact double value of an f32 scalar."""
    return float(np.float32(v))


def read_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals, tol = (s.strip() for s in line.split("|"))
            out[key] = (np.array([float(v) for v in vals.split()]), float(tol))
    return out


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.maximum(np.abs(b), 1e-300)
    return np.where(b == 0, np.abs(a), np.abs(a - b) / den)


# ---------------------------------------------------------------------------
# Page-printed values
# ---------------------------------------------------------------------------

def pin_worked_example(O):
    g = read_golden("rmsnorm_worked_example.txt")
    x = g["x"][0].astype(F32)[None, :]
    eps = float(g["eps"][0][0])
    for gkey, ykey in (("gamma_one", "y_one"), ("gamma_two", "y_two")):
        gamma = g[gkey][0].astype(F32)
        y, rms = O.rmsnorm(x, gamma, eps, return_rms=True)
        want, tol = g[ykey]
        assert np.all(np.abs(y[0] - want) <= tol), (ykey, y[0], want)
        zero = want == 0
        assert np.all(y[0][zero] == 0.0), "zeros of the example must be exact"
        r, rtol = g["rms"]
        assert abs(rms[0] - r[0]) <= rtol, ("rms", rms[0])
        inv, itol = g["inv_rms"]
        assert abs(1.0 / rms[0] - inv[0]) <= itol, ("inv_rms", 1 / rms[0])
    y1 = O.rmsnorm(x, g["gamma_one"][0].astype(F32), eps)
    m, mtol = g["mean_y_sq"]
    assert abs(np.mean(y1[0] ** 2) - m[0]) <= mtol


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def pin_constant_rows(O):
    """x = c everywhere: mean(x^2) = c^2, so y_j = gamma_j c / sqrt(c^2 + eps)."""
    rng = rng_for(11)
    for n in (1, 2, 3, 7, 100, 1000):
        gamma = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        for c in (1.5, -1.5, 3.0e-4, -7.0e3, 2.0 ** -20, 1e18):
            for eps in (1e-5, 1e-8, 1e-6):
                x = np.full((1, n), c, F32)
                y = O.rmsnorm(x, gamma, eps)[0]
                cf, ef = _f(c), _f(eps)
                want = gamma.astype(np.float64) * (cf / math.sqrt(cf * cf + ef))
                # f64 sequential sum of n equal squares: relative error of the
                # sum <= (n - 1) u, halved by the root, plus a few roundings
                bound = (n + 8) * 2.0 ** -53
                assert np.max(_rel(y, want)) < bound, (n, c, eps)


def pin_zero_rows(O):
    """A zero row normalises to exactly zero (eps keeps the root positive);
    in the tail, a = 0 or gamma_post = 0 leaves h = r exactly."""
    rng = rng_for(12)
    for n in (1, 2, 5, 64):
        gamma = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        y = O.rmsnorm(np.zeros((3, n), F32), gamma, 1e-5)
        assert np.all(y == 0.0) and np.all(np.isfinite(y))
        r = rng.standard_normal((2, n)).astype(F32)
        a = rng.standard_normal((2, n)).astype(F32)
        gq = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        plain_r = O.rmsnorm(r, gq, 1e-5)
        for aa, gp in ((np.zeros_like(a), gamma), (a, np.zeros(n, F32))):
            t = O.sandwich_tail(aa, r, gp, 1e-8, gq, 1e-5)
            assert np.array_equal(t.h, r.astype(np.float64))
            assert np.array_equal(t.p, np.zeros_like(t.p))
            assert np.max(_rel(t.y, plain_r)) < 1e-15


def pin_n1(O):
    """n = 1: y = gamma x / sqrt(x^2 + eps)."""
    for xv in (0.5, -3.0, 1e-4, 1e-3, 123.25):
        for eps in (1e-5, 1e-8):
            y = O.rmsnorm(np.array([[xv]], F32), np.array([0.75], F32), eps)
            xf = _f(xv)
            want = 0.75 * xf / math.sqrt(xf * xf + _f(eps))
            assert abs(y[0, 0] - want) <= 1e-15 * abs(want), (xv, eps)


def pin_hand_n2(O):
    """Hand-worked n = 2 rows (unit gain, eps = 1e-5 as f32)."""
    e = _f(1e-5)
    t = _f(1e-3)
    cases = [
        ([3.0, 4.0], [3 / math.sqrt(12.5 + e), 4 / math.sqrt(12.5 + e)]),
        ([1.0, -1.0], [1 / math.sqrt(1 + e), -1 / math.sqrt(1 + e)]),
        ([1.0, 0.0], [math.sqrt(2) / math.sqrt(1 + 2 * e), 0.0]),
        ([t, t], [1 / math.sqrt(1 + e / (t * t))] * 2),
        ([0.0, 0.0], [0.0, 0.0]),
    ]
    gamma = np.ones(2, F32)
    for xs, want in cases:
        y = O.rmsnorm(np.array([xs], F32), gamma, 1e-5)[0]
        assert np.max(_rel(y, want)) < 2e-15, (xs, y, want)
    # the epsilon-dominated [1e-3, 1e-3] row is far from unit scale: with
    # decimal inputs it would be 1/sqrt(11); the f32 rounding of 1e-3 and 1e-5
    # moves it by about 1.6e-8
    y = O.rmsnorm(np.array([[t, t]], F32), gamma, 1e-5)[0]
    assert abs(y[0] - 1 / math.sqrt(11)) < 3e-8


def pin_tail_hand_example(O):
    """a = [3, 4], r = [1, -1], unit gains, eps_post = 1e-8, eps_pre = 1e-5."""
    ep, eq = _f(1e-8), _f(1e-5)
    d_a = math.sqrt(12.5 + ep)
    p = [3 / d_a, 4 / d_a]
    h = [1 + p[0], -1 + p[1]]
    d_h = math.sqrt((h[0] ** 2 + h[1] ** 2) / 2 + eq)
    y = [h[0] / d_h, h[1] / d_h]
    one = np.ones(2, F32)
    t = O.sandwich_tail(np.array([[3, 4]], F32), np.array([[1, -1]], F32),
                        one, 1e-8, one, 1e-5)
    scale = np.abs([1.0, -1.0]) + np.abs(p)
    assert np.max(_rel(t.p[0], p)) < 2e-15
    assert np.all(np.abs(t.h[0] - h) <= 2e-15 * scale)
    assert np.all(np.abs(t.y[0] - y) <= 4e-15 * scale / d_h)
    assert abs(t.d_a[0] - d_a) < 1e-15 and abs(t.d_h[0] - d_h) < 1e-15
    # worked through by hand to 12 digits
    assert abs(t.h[0, 0] - 1.848528137084) < 1e-11
    assert abs(t.h[0, 1] - 0.131370849446) < 1e-11
    assert abs(t.y[0, 0] - 1.410651588865) < 1e-11
    assert abs(t.y[0, 1] - 0.100251921398) < 1e-11


def pin_eps_dominated(O):
    """mean(x^2) = m << eps: y / (gamma x / sqrt(eps)) = (1 + m/eps)^(-1/2)
    = 1 - m/(2 eps) + O((m/eps)^2)."""
    rng = rng_for(13)
    for eps in (1e-5, 1e-8, 1e-6):
        for n in (2, 16, 300):
            x = (rng.standard_normal((1, n)) * math.sqrt(eps) * 1e-3).astype(F32)
            gamma = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
            y = O.rmsnorm(x, gamma, eps)[0]
            xd = x[0].astype(np.float64)
            m = float(np.mean(xd * xd))
            ratio = y / (gamma * xd / math.sqrt(_f(eps)))
            t = m / _f(eps)
            assert t < 1e-5
            assert np.max(np.abs(ratio - (1 - t / 2))) <= t * t + 1e-15, eps


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def pin_unit_gain_mean_square(O):
    """gamma = 1: mean(y^2) = m / (m + eps) with m = mean(x^2) (rms(y) = 1 in
    the limit eps -> 0, the page's check after Figure 12.1)."""
    rng = rng_for(14)
    for n in (3, 64, 6656):
        for lg in (-6, -2, 0, 3):
            x = (rng.standard_normal((2, n)) * 10.0 ** lg).astype(F32)
            y = O.rmsnorm(x, np.ones(n, F32), 1e-5)
            xd = x.astype(np.float64)
            m = np.mean(xd * xd, axis=1)
            want = m / (m + _f(1e-5))
            got = np.mean(y * y, axis=1)
            assert np.max(_rel(got, want)) < 1e-13, (n, lg)


def pin_scale_invariance(O):
    """y(alpha x; eps) = y(x; eps / alpha^2) exactly for alpha a power of two
    (every operation scales exactly), and y(alpha x) ~ y(x) when eps << m."""
    rng = rng_for(15)
    for n in (2, 5, 513):
        x = (rng.standard_normal((3, n)) * 0.5).astype(F32)
        gamma = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        eps = 2.0 ** -17
        for k in (-20, -3, 5, 30):
            alpha = 2.0 ** k
            y1 = O.rmsnorm((x * F32(alpha)).astype(F32), gamma, eps)
            y2 = O.rmsnorm(x, gamma, eps / alpha ** 2)
            assert np.array_equal(y1, y2), (n, k)
        # eps negligible: plain scale invariance up to ~eps/m
        xd = x.astype(np.float64)
        m = np.mean(xd * xd, axis=1, keepdims=True)
        ya = O.rmsnorm((x * F32(1024.0)).astype(F32), gamma, 1e-8)
        yb = O.rmsnorm(x, gamma, 1e-8)
        assert np.all(np.abs(ya - yb) <= (1e-8 / m + 1e-15) * np.abs(yb) + 1e-15)


def pin_row_independence(O):
    """A batch of rows equals each row normalised on its own (row stride n)."""
    rng = rng_for(16)
    for n in (1, 3, 8, 77):
        x = rng.standard_normal((5, n)).astype(F32)
        gamma = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        yb = O.rmsnorm(x, gamma, 1e-5)
        for i in range(5):
            assert np.array_equal(yb[i], O.rmsnorm(x[i:i + 1], gamma, 1e-5)[0])
        a = rng.standard_normal((4, n)).astype(F32)
        r = rng.standard_normal((4, n)).astype(F32)
        tb = O.sandwich_tail(a, r, gamma, 1e-8, gamma[::-1].copy(), 1e-5)
        for i in range(4):
            ti = O.sandwich_tail(a[i:i + 1], r[i:i + 1], gamma, 1e-8,
                                 gamma[::-1].copy(), 1e-5)
            assert np.array_equal(tb.h[i], ti.h[0])
            assert np.array_equal(tb.y[i], ti.y[0])


# ---------------------------------------------------------------------------
# Library routines
# ---------------------------------------------------------------------------

def pin_torch_rms_norm(O):
    import torch
    import torch.nn.functional as F
    rng = rng_for(17)
    for n, lg in ((4, 0), (128, -3), (6656, 1), (6657, -5), (2, 2)):
        x = (rng.standard_normal((6, n)) * 10.0 ** lg).astype(F32)
        gamma = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        for eps in (1e-5, 1e-8):
            want = F.rms_norm(torch.from_numpy(x).double(), (n,),
                              torch.from_numpy(gamma).double(),
                              eps=_f(eps)).numpy()
            got = O.rmsnorm(x, gamma, eps)
            assert np.max(_rel(got, want)) < 1e-13, (n, eps)


def pin_layer_norm_identity(O):
    """On rows whose mean is exactly zero, LayerNorm without bias equals
    RMSNorm. Rows are symmetric multisets of multiples of 1/16, so every sum is
    exact in f64 whatever order a library adds in."""
    import torch
    import torch.nn.functional as F
    rng = rng_for(18)
    for half in (1, 3, 50, 2000):
        k = rng.integers(-100, 101, half)
        vals = np.concatenate([k, -k]) / 16.0
        x = rng.permutation(vals).astype(F32)[None, :]
        n = x.shape[1]
        gamma = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        for eps in (1e-5, 1e-8):
            want = F.layer_norm(torch.from_numpy(x).double(), (n,),
                                torch.from_numpy(gamma).double(), None,
                                eps=_f(eps)).numpy()
            got = O.rmsnorm(x, gamma, eps)
            assert np.max(_rel(got, want)) < 1e-13, (n, eps)


# ---------------------------------------------------------------------------
# Exact arithmetic on tiny inputs
# ---------------------------------------------------------------------------

def _dec_rms(xs, gs, eps):
    n = len(xs)
    s = sum((x * x for x in xs), Decimal(0))
    rms = (s / Decimal(n) + eps).sqrt()
    return [x / rms * g for x, g in zip(xs, gs)], rms


def _tiny_rows(rng, count, nmax):
    rows = []
    for i in range(count):
        n = int(rng.integers(1, nmax + 1))
        lg = rng.uniform(-5, 3)
        rows.append((rng.standard_normal(n) * 10.0 ** lg).astype(F32))
    return rows


def pin_decimal_plain(O):
    getcontext().prec = 50
    rng = rng_for(19)
    for x in _tiny_rows(rng, 60, 16):
        n = x.size
        gamma = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        for eps in (1e-5, 1e-8):
            want, _ = _dec_rms([Decimal(float(v)) for v in x],
                               [Decimal(float(v)) for v in gamma],
                               Decimal(_f(eps)))
            got = O.rmsnorm(x[None, :], gamma, eps)[0]
            want = np.array([float(w) for w in want])
            assert np.max(_rel(got, want)) < 1e-14, (n, eps)


def pin_decimal_bf16(O):
    """bf16 storage is decoded exactly: the bf16 result equals the exact value
    on the decoded inputs, and equals the f32 path on the same values."""
    getcontext().prec = 50
    rng = rng_for(20)
    for x in _tiny_rows(rng, 40, 16):
        n = x.size
        xb = f32_to_bf16_bits(x)
        gb = f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(n)).astype(F32))
        xd, gd = bf16_bits_to_f32(xb), bf16_bits_to_f32(gb)
        want, _ = _dec_rms([Decimal(float(v)) for v in xd],
                           [Decimal(float(v)) for v in gd], Decimal(_f(1e-6)))
        got = O.rmsnorm(xb[None, :], gb, 1e-6)[0]
        want = np.array([float(w) for w in want])
        assert np.max(_rel(got, want)) < 1e-14
        assert np.array_equal(got, O.rmsnorm(xd[None, :], gd, 1e-6)[0])


def pin_decimal_tail(O):
    """Exact fused tail. Rows are drawn so that mean(a^2) sits near eps_post
    and mean(h^2) near eps_pre in some rows: swapping or dropping either
    epsilon changes those rows by far more than the tolerance."""
    getcontext().prec = 50
    rng = rng_for(21)
    ep, eq = Decimal(_f(1e-8)), Decimal(_f(1e-5))
    for i in range(60):
        n = int(rng.integers(1, 17))
        a_lg = rng.choice([-4.0, -4.5, -2.0, 0.0, 1.5])
        r_lg = rng.choice([-3.0, -2.5, -1.0, 0.5])
        a = (rng.standard_normal(n) * 10.0 ** a_lg).astype(F32)
        r = (rng.standard_normal(n) * 10.0 ** r_lg).astype(F32)
        gp = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        gq = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        ad = [Decimal(float(v)) for v in a]
        p, d_a = _dec_rms(ad, [Decimal(float(v)) for v in gp], ep)
        h = [Decimal(float(rv)) + pv for rv, pv in zip(r, p)]
        y, d_h = _dec_rms(h, [Decimal(float(v)) for v in gq], eq)
        t = O.sandwich_tail(a[None, :], r[None, :], gp, 1e-8, gq, 1e-5)
        scale = np.abs(r.astype(np.float64)) + np.abs([float(v) for v in p])
        hw = np.array([float(v) for v in h])
        yw = np.array([float(v) for v in y])
        assert np.all(np.abs(t.h[0] - hw) <= 1e-14 * scale + 1e-300), i
        yscale = np.abs(gq.astype(np.float64)) * scale / float(d_h)
        assert np.all(np.abs(t.y[0] - yw) <= 1e-14 * yscale + 1e-300), i
        assert abs(t.d_a[0] - float(d_a)) <= 1e-14 * float(d_a)
        assert abs(t.d_h[0] - float(d_h)) <= 1e-14 * float(d_h)


# ---------------------------------------------------------------------------
# The tail's two halves (Hesper "RMSNorm Layer": rmsNormThenAdd[...]Kernel,
# residualAddRmsNormKernel)
# ---------------------------------------------------------------------------

def pin_norm_then_add_closed_forms(O):
    """a = 0 gives out = r * scale exactly; r = 0 gives rmsnorm(a) * scale;
    the hand example a = [3, 4], r = [1, -1], scale 2."""
    rng = rng_for(31)
    for n in (1, 2, 7, 130):
        g = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        r = rng.standard_normal((3, n)).astype(F32)
        a = (rng.standard_normal((3, n)) * 10).astype(F32)
        for scale in (None, 2.0, -0.5):
            sc = 1.0 if scale is None else scale
            out, _ = O.norm_then_add(np.zeros_like(a), r, g, 1e-8, scale)
            assert np.array_equal(out, r.astype(np.float64) * sc)
            out, _ = O.norm_then_add(a, np.zeros_like(r), g, 1e-8, scale)
            assert np.array_equal(out, O.rmsnorm(a, g, 1e-8) * sc)
    ep = _f(1e-8)
    d = math.sqrt(12.5 + ep)
    want = [(3 / d + 1) * 2, (4 / d - 1) * 2]
    out, dd = O.norm_then_add(np.array([[3, 4]], F32),
                              np.array([[1, -1]], F32), np.ones(2, F32), 1e-8,
                              2.0)
    assert np.all(np.abs(out[0] - want) <= 4e-15 * (np.abs(want) + 2))
    assert abs(dd[0] - d) <= 1e-15 * d
    assert abs(out[0, 0] - 3.697056274168) < 1e-11


def pin_add_then_norm_closed_forms(O):
    """b = 0 gives s = a and y = rmsnorm(a) exactly; b = -a gives zeros; the
    hand example a = [3, 4], b = [1, -1] (s = [4, 3])."""
    rng = rng_for(32)
    for n in (1, 3, 64):
        g = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        a = (rng.standard_normal((2, n)) * 3).astype(F32)
        s, y, _ = O.add_then_norm(a, np.zeros_like(a), g, 1e-5)
        assert np.array_equal(s, a.astype(np.float64))
        assert np.array_equal(y, O.rmsnorm(a, g, 1e-5))
        s, y, _ = O.add_then_norm(a, -a, g, 1e-5)
        assert np.all(s == 0) and np.all(y == 0)
    e = _f(1e-5)
    d = math.sqrt(12.5 + e)
    s, y, dd = O.add_then_norm(np.array([[3, 4]], F32),
                               np.array([[1, -1]], F32), np.ones(2, F32), 1e-5)
    assert np.array_equal(s[0], [4.0, 3.0])
    assert np.max(_rel(y[0], [4 / d, 3 / d])) < 2e-15
    assert abs(y[0, 0] - 1.131370397350) < 1e-11


def pin_halves_compose_to_the_tail(O):
    """The tail's h is norm_then_add(a, r) with the post-norm gain and
    epsilon; add_then_norm on an exactly representable sum equals rmsnorm of
    that sum."""
    rng = rng_for(33)
    for n in (2, 9, 300):
        a = rng.standard_normal((4, n)).astype(F32)
        r = rng.standard_normal((4, n)).astype(F32)
        gp = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        gq = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        t = O.sandwich_tail(a, r, gp, 1e-8, gq, 1e-5)
        out, d = O.norm_then_add(a, r, gp, 1e-8)
        assert np.array_equal(out, t.h) and np.array_equal(d, t.d_a)
        ai = rng.integers(-50, 50, (3, n)).astype(F32)
        bi = rng.integers(-50, 50, (3, n)).astype(F32)
        s, y, _ = O.add_then_norm(ai, bi, gq, 1e-5)
        assert np.array_equal(y, O.rmsnorm((ai + bi).astype(F32), gq, 1e-5))


def pin_halves_torch(O):
    import torch
    import torch.nn.functional as F
    rng = rng_for(34)
    for n in (5, 128, 6656):
        a = (rng.standard_normal((3, n)) * 10.0 ** rng.uniform(-3, 2)).astype(F32)
        b = rng.standard_normal((3, n)).astype(F32)
        g = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        tg = torch.from_numpy(g).double()
        ta, tb = torch.from_numpy(a).double(), torch.from_numpy(b).double()
        want = (F.rms_norm(ta, (n,), tg, eps=_f(1e-8)) + tb) * 0.75
        out, _ = O.norm_then_add(a, b, g, 1e-8, 0.75)
        assert np.max(np.abs(out - want.numpy()) /
                      (np.abs(want.numpy()) + 1.0)) < 1e-13
        s, y, _ = O.add_then_norm(a, b, g, 1e-5)
        want = F.rms_norm(ta + tb, (n,), tg, eps=_f(1e-5)).numpy()
        assert np.max(_rel(y, want)) < 1e-12


def pin_decimal_halves(O):
    getcontext().prec = 50
    rng = rng_for(35)
    for i in range(40):
        n = int(rng.integers(1, 17))
        a = (rng.standard_normal(n) * 10.0 ** rng.choice([-4.0, -2.0, 0.0, 1.0])
             ).astype(F32)
        r = (rng.standard_normal(n) * 10.0 ** rng.choice([-3.0, -1.0, 0.5])
             ).astype(F32)
        g = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        scale = float(rng.choice([1.0, 0.5, 3.0]))
        eps = float(rng.choice([1e-8, 1e-5]))
        ad = [Decimal(float(v)) for v in a]
        rd = [Decimal(float(v)) for v in r]
        gd = [Decimal(float(v)) for v in g]
        p, _ = _dec_rms(ad, gd, Decimal(_f(eps)))
        want = np.array([float((pv + rv) * Decimal(scale))
                         for pv, rv in zip(p, rd)])
        out, _ = O.norm_then_add(a[None, :], r[None, :], g, eps, scale)
        sc = (np.abs([float(v) for v in p]) + np.abs(r)) * abs(scale)
        assert np.all(np.abs(out[0] - want) <= 1e-14 * sc + 1e-300), i
        sd = [x + y for x, y in zip(ad, rd)]
        yd, dd = _dec_rms(sd, gd, Decimal(_f(eps)))
        s, y, d = O.add_then_norm(a[None, :], r[None, :], g, eps)
        sc = np.abs(a.astype(np.float64)) + np.abs(r)
        assert np.all(np.abs(s[0] - np.array([float(v) for v in sd]))
                      <= 1e-15 * sc), i
        ysc = np.abs(g.astype(np.float64)) * sc / float(dd)
        assert np.all(np.abs(y[0] - np.array([float(v) for v in yd]))
                      <= 1e-14 * ysc + 1e-300), i
        assert abs(d[0] - float(dd)) <= 1e-14 * float(dd)


# ---------------------------------------------------------------------------
# RMSNorm + Q8_1 (Hesper "RMSNorm Layer", Fused RMSNorm + Q8_1 quantize)
# ---------------------------------------------------------------------------

def _near_tie(t, band=1e-9):
    f = np.abs(np.asarray(t) - np.floor(t) - 0.5)
    return f < band


def pin_q8_closed_form(O):
    """gamma = 1, block x = 1..32: q_j = round(127 j / 32) (ties to even;
    the tie at j = 16 is not decided here, see _near_tie), and
    d = 32 / sqrt(357.5 + eps) / 127 since mean(j^2) = 33 * 65 / 6."""
    x = np.arange(1, 33, dtype=F32)[None, :]
    y, d, t, q = O.rmsnorm_q8_1(x, np.ones(32, F32), 1e-5)
    want_t = 127.0 * np.arange(1, 33) / 32.0
    ok = ~_near_tie(want_t)
    assert np.all(q[0][ok] == np.array([round(v) for v in want_t])[ok])
    assert np.max(np.abs(t[0] - want_t)) < 1e-12
    wd = 32.0 / math.sqrt(357.5 + _f(1e-5)) / 127.0
    assert abs(d[0, 0] - wd) < 1e-15
    # negated row: negated codes
    _, _, _, qn = O.rmsnorm_q8_1(-x, np.ones(32, F32), 1e-5)
    assert np.array_equal(qn[0][ok], -q[0][ok])


def pin_q8_properties(O):
    """Every nonzero block reaches |q| = 127 at its largest value; d * q is
    within d / 2 of the normalised value; a zero block encodes as d = 0,
    q = 0; codes do not depend on the row's scale (inv_rms cancels in
    x_normed / d)."""
    rng = rng_for(41)
    for n in (32, 64, 320):
        x = (rng.standard_normal((6, n)) * 10.0 ** rng.uniform(-3, 3, (6, 1))
             ).astype(F32)
        x[2, 32:64] = 0.0 if n >= 64 else x[2, 32:64]
        g = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        y, d, t, q = O.rmsnorm_q8_1(x, g, 1e-5)
        nb = n // 32
        qb = q.reshape(6, nb, 32).astype(np.int32)
        yb = y.reshape(6, nb, 32)
        for i in range(6):
            for b in range(nb):
                if np.all(yb[i, b] == 0):
                    assert d[i, b] == 0 and np.all(qb[i, b] == 0)
                    continue
                assert np.max(np.abs(qb[i, b])) == 127
                assert np.all(np.abs(d[i, b] * qb[i, b] - yb[i, b]) <=
                              d[i, b] * (0.5 + 1e-9))
        y2, d2, t2, q2 = O.rmsnorm_q8_1((x * F32(8.0)).astype(F32), g, 1e-5)
        ok = ~_near_tie(t) & ~_near_tie(t2)
        assert np.array_equal(q[ok], q2[ok])


def pin_q8_ties_to_even(O):
    """Exact ties: x = [254, 1, 3, 5, 7, -1, -3, -5, -7, 200, 160, 28, 2,
    0 x 19], gamma = 1, eps = 1e-30. Sum x^2 = 131072 = 32 * 4096, so
    mean + eps rounds to 4096 and rms = 64 exactly; y = x / 64 exactly,
    amax = 254 / 64 and d = amax / 127 = 1 / 32 exactly, so t = x / 2
    exactly and the odd entries are true ties k + 1/2. Round half to even
    (WGSL round) gives 0, 2, 2, 4 for 0.5, 1.5, 2.5, 3.5; half away from
    zero would give 1, 2, 3, 4."""
    vals = [254, 1, 3, 5, 7, -1, -3, -5, -7, 200, 160, 28, 2] + [0] * 19
    assert sum(v * v for v in vals) == 32 * 4096
    x = np.array([vals], F32)
    y, d, t, q = O.rmsnorm_q8_1(x, np.ones(32, F32), 1e-30)
    assert d[0, 0] == 1.0 / 32.0
    assert np.array_equal(t[0], np.array(vals, np.float64) / 2.0)
    want = [127, 0, 2, 2, 4, 0, -2, -2, -4, 100, 80, 14, 1] + [0] * 19
    assert q[0].tolist() == want


def pin_q8_decimal(O):
    """Exact decimal arithmetic on short rows: codes agree away from ties,
    scales to 1e-14."""
    from decimal import ROUND_HALF_EVEN
    getcontext().prec = 50
    rng = rng_for(42)
    for it in range(12):
        n = 32 * int(rng.integers(1, 4))
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-2, 2)).astype(F32)
        g = (1 + 0.1 * rng.standard_normal(n)).astype(F32)
        yd, _ = _dec_rms([Decimal(float(v)) for v in x],
                         [Decimal(float(v)) for v in g], Decimal(_f(1e-5)))
        y, d, t, q = O.rmsnorm_q8_1(x[None, :], g, 1e-5)
        for b in range(n // 32):
            blk = yd[b * 32:(b + 1) * 32]
            amax = max(abs(v) for v in blk)
            db = amax / Decimal(127)
            assert abs(d[0, b] - float(db)) <= 1e-14 * float(db)
            for l, v in enumerate(blk):
                tv = v / db
                frac = abs(tv - tv.to_integral_value(rounding="ROUND_FLOOR")
                           - Decimal("0.5"))
                if frac < Decimal("1e-9"):
                    continue
                qv = int(tv.to_integral_value(rounding=ROUND_HALF_EVEN))
                assert q[0, b * 32 + l] == max(-128, min(127, qv)), (it, b, l)


ALL_PINS = [
    pin_worked_example,
    pin_constant_rows,
    pin_zero_rows,
    pin_n1,
    pin_hand_n2,
    pin_tail_hand_example,
    pin_eps_dominated,
    pin_unit_gain_mean_square,
    pin_scale_invariance,
    pin_row_independence,
    pin_torch_rms_norm,
    pin_layer_norm_identity,
    pin_decimal_plain,
    pin_decimal_bf16,
    pin_decimal_tail,
    pin_norm_then_add_closed_forms,
    pin_add_then_norm_closed_forms,
    pin_halves_compose_to_the_tail,
    pin_halves_torch,
    pin_decimal_halves,
    pin_q8_closed_form,
    pin_q8_properties,
    pin_q8_ties_to_even,
    pin_q8_decimal,
]
