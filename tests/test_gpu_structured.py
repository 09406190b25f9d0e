"""Structured rows through every operation and storage type, against the
oracle: zero rows, constant rows, alternating signs, a one-hot spike, rows
at the bottom of the tested range, exact cancellation of the residual add
(a = -b for add_then_norm) and near-complete cancellation in the tail (a
row of ones with r = -a and a unit gain). The edge sweep covers these shapes
for the plain f32 norm only; here each operation meets them in f32, bf16 and
f16, at a narrow and at the model's width."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import (check_add_norm, check_norm_add, check_plain,  # noqa: E402
                         check_q8, check_tail, run_add_norm, run_norm_add,
                         run_plain, run_q8, run_tail, say)

pytestmark = pytest.mark.gpu

KINDS = ["zero", "constant", "alternating", "spike", "tiny", "random"]


def structured(kind, rows, n, rng, scale=1.0):
    """[rows, n] float32 rows of one structure (row i varies the value)."""
    x = np.empty((rows, n), np.float64)
    for i in range(rows):
        c = scale * (0.5 + i) * (-1) ** i
        if kind == "zero":
            x[i] = 0.0
        elif kind == "constant":
            x[i] = c
        elif kind == "alternating":
            x[i] = np.where(np.arange(n) % 2 == 0, c, -c)
        elif kind == "spike":
            x[i] = 0.0
            x[i, (7 * i) % n] = 100.0 * c
        elif kind == "tiny":
            x[i] = 1e-6 * scale * rng.standard_normal(n)
        else:
            x[i] = scale * rng.standard_normal(n)
    return x.astype(np.float32)


def _st(x, dtype):
    return gen.to_storage(x, dtype)


def _gain(rng, n, dtype):
    return _st((1.0 + 0.1 * rng.standard_normal(n)).astype(np.float32), dtype)


CASES = [(op, dtype, n, kind)
         for op in ("plain", "tail", "norm_add", "add_norm", "q8")
         for dtype in ("f32", "bf16", "f16")
         for n in (96, 6656)
         for kind in KINDS]


@pytest.mark.parametrize("case", CASES,
                         ids=["-".join(map(str, c)) for c in CASES])
def test_structured_rows(oracle, case):
    op, dtype, n, kind = case
    label = f"structured {op} {dtype} n={n} {kind}"
    say(label)
    rng = gen.rng_for(40000 + 97 * KINDS.index(kind) + n)
    rows = 6
    if op in ("plain", "q8"):
        inp = {"x": _st(structured(kind, rows, n, rng), dtype),
               "gamma": _gain(rng, n, dtype), "eps": 1e-5, "dtype": dtype}
        if op == "plain":
            got, _ = run_plain(inp)
            check_plain(oracle, inp, got, label)
        else:
            check_q8(oracle, inp, run_q8(inp), label)
    elif op == "tail":
        a = structured(kind, rows, n, rng)
        r = structured(KINDS[(KINDS.index(kind) + 1) % len(KINDS)], rows, n,
                       rng, scale=3.0)
        gp = _gain(rng, n, dtype)
        if kind == "constant":
            # r = -a with a unit gain: h = sign(a) (1 - |a|) up to epsilon,
            # which cancels almost completely in the row of ones
            a[0] = 1.0
            r = -a
            gp = _st(np.ones(n, np.float32), dtype)
        inp = {"a": _st(a, dtype), "r": _st(r, dtype), "gamma_post": gp,
               "gamma_pre": _gain(rng, n, dtype), "eps_post": 1e-8,
               "eps_pre": 1e-5, "dtype": dtype}
        h, y = run_tail(inp)
        check_tail(oracle, inp, h, y, label)
    elif op == "norm_add":
        a = structured(kind, rows, n, rng)
        b = structured(KINDS[(KINDS.index(kind) + 2) % len(KINDS)], rows, n,
                       rng, scale=2.0)
        inp = {"a": _st(a, dtype), "b": _st(b, dtype),
               "gamma": _gain(rng, n, dtype), "eps": 1e-8, "dtype": dtype}
        check_norm_add(oracle, inp, run_norm_add(inp), None, label)
    else:
        a = structured(kind, rows, n, rng)
        b = -a if kind in ("constant", "alternating") else \
            structured(KINDS[(KINDS.index(kind) + 3) % len(KINDS)], rows, n,
                       rng, scale=0.5)
        inp = {"a": _st(a, dtype), "b": _st(b, dtype),
               "gamma": _gain(rng, n, dtype), "eps": 1e-5, "dtype": dtype}
        s, y = run_add_norm(inp)
        check_add_norm(oracle, inp, s, y, label)
        if kind in ("constant", "alternating"):
            # a + b = 0 exactly: the sum and y are exactly zero
            assert not s.any() and not y.any()
