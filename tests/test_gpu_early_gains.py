"""Row-tile launches of at most 16 rows load the gains together with the row;
longer launches load each gain vector just before its use. Only the time a
load is issued differs, not the arithmetic, so the two forms must agree bit
for bit.

For each row tile that has both forms (one row per workgroup, at most four
vectors per lane), forced, with a ragged row that fills the tile: 40 rows in
one launch (gains loaded late) against the same rows in launches of 16, 7
and 1 rows (gains loaded with the row) and of the 16 rows left (late again)
on slices of the same buffers. Every slice must equal the matching rows of
the 40-row launch, and the 16-row launch is also checked against the
oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import (check_add_norm, check_plain, check_tail, dev,  # noqa: E402
                         host_f64, say)

pytestmark = pytest.mark.gpu

ROWS = 40
PIECES = ((0, 16), (16, 23), (23, 24), (24, 40))   # 16, 7, 1, 16 rows
TILES = ((128, 2), (256, 2), (256, 4), (512, 2), (512, 4), (1024, 1),
         (1024, 2), (1024, 4))
WIDTH = {"f32": 4, "bf16": 8, "f16": 8}

CASES = [(op, dtype, g, vpt)
         for op in ("plain", "tail", "add_norm")
         for dtype in ("f32", "bf16", "f16")
         for g, vpt in TILES]


def _gain(rng, n, dtype):
    return gen.to_storage((1.0 + 0.1 * rng.standard_normal(n))
                          .astype(np.float32), dtype)


def _rows(rng, n, dtype, scale=1.0):
    return gen.to_storage((scale * rng.standard_normal((ROWS, n)))
                          .astype(np.float32), dtype)


def _call(op, ins, outs, lo, hi, eps):
    """One launch over rows [lo, hi) of the device buffers."""
    sl = [t[lo:hi] for t in ins]
    ol = [t[lo:hi] for t in outs]
    if op == "plain":
        snr.rmsnorm_fwd(sl[0], ins[1], eps[0], out=ol[0])
    elif op == "tail":
        snr.sandwich_tail(sl[0], sl[1], ins[2], eps[0], ins[3], eps[1],
                          h_out=ol[0], y_out=ol[1])
    else:
        snr.add_then_norm(sl[0], sl[1], ins[2], eps[0], sum_out=ol[0],
                          y_out=ol[1])


@pytest.mark.parametrize("case", CASES,
                         ids=["-".join(map(str, c)) for c in CASES])
def test_early_and_late_gains_agree(oracle, case):
    op, dtype, g, vpt = case
    n = g * vpt * WIDTH[dtype] - 3        # the tile's last vector ragged
    label = f"early-gains {op} {dtype} rowtile {g}x{vpt} n={n}"
    say(label)
    rng = gen.rng_for(60000 + 31 * g + vpt + 7 * n)
    if op == "plain":
        inp = {"x": _rows(rng, n, dtype), "gamma": _gain(rng, n, dtype),
               "eps": 1e-5, "dtype": dtype}
        ins = [dev(inp["x"], dtype)]
        eps = (inp["eps"],)
        keys = ("gamma",)
    elif op == "tail":
        inp = {"a": _rows(rng, n, dtype), "r": _rows(rng, n, dtype, 3.0),
               "gamma_post": _gain(rng, n, dtype),
               "gamma_pre": _gain(rng, n, dtype), "eps_post": 1e-8,
               "eps_pre": 1e-5, "dtype": dtype}
        ins = [dev(inp["a"], dtype), dev(inp["r"], dtype)]
        eps = (inp["eps_post"], inp["eps_pre"])
        keys = ("gamma_post", "gamma_pre")
    else:
        inp = {"a": _rows(rng, n, dtype), "b": _rows(rng, n, dtype, 0.5),
               "gamma": _gain(rng, n, dtype), "eps": 1e-5, "dtype": dtype}
        ins = [dev(inp["a"], dtype), dev(inp["b"], dtype)]
        eps = (inp["eps"],)
        keys = ("gamma",)
    ins += [dev(inp[k], dtype) for k in keys]
    outs_n = 1 if op == "plain" else 2
    whole = [torch.full_like(ins[0], float("nan")) for _ in range(outs_n)]
    parts = [torch.full_like(ins[0], float("nan")) for _ in range(outs_n)]
    with snr.forced_shape("rowtile", g, vpt):
        _call(op, ins, whole, 0, ROWS, eps)
        assert snr.last_shape() == f"rowtile:{g}:{vpt}:{WIDTH[dtype]}", \
            snr.last_shape()
        for lo, hi in PIECES:
            _call(op, ins, parts, lo, hi, eps)
    torch.cuda.synchronize()
    for w, p in zip(whole, parts):
        assert torch.equal(w.view(torch.int16 if dtype != "f32"
                                  else torch.int32),
                           p.view(torch.int16 if dtype != "f32"
                                  else torch.int32)), label

    # the first 16-row launch against the oracle
    lo, hi = PIECES[0]
    sub = {k: (v[lo:hi] if isinstance(v, np.ndarray) and v.ndim == 2 else v)
           for k, v in inp.items()}
    got = [host_f64(p[lo:hi]) for p in parts]
    if op == "plain":
        check_plain(oracle, sub, got[0], label)
    elif op == "tail":
        check_tail(oracle, sub, got[0], got[1], label)
    else:
        check_add_norm(oracle, sub, got[0], got[1], label)
