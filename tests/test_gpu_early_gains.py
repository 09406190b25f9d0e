"""Row-tile launches of at most 16 workgroups load the gains together with
the row; larger launches load each gain vector just before its use. Only the
time a load is issued differs, not the arithmetic, so the two forms must
agree bit for bit.

For each row tile that has both forms (at most four vectors per lane;
sub-wavefront tiles included, whose 256-lane workgroups hold 256 / G rows),
forced, with a ragged row that fills the tile: 26 workgroups' worth of rows
in one launch (gains loaded late) against the same rows in launches of 16
workgroups, 7 rows, 1 row and the rest (gains loaded with the row) on slices
of the same buffers. Every slice must equal the matching rows of the whole
launch, and the first slice is also checked against the oracle. The
several-segment launch is checked the same way: two segments in one launch
of 52 workgroups against their first rows in a launch of 16."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import (check_add_norm, check_norm_add, check_plain,  # noqa: E402
                         check_tail, dev, host_f64, run_add_norm,
                         run_norm_add, run_plain, run_tail, say)

pytestmark = pytest.mark.gpu

EARLY_BLOCKS = 16
TILES = ((1, 4), (2, 4), (4, 4), (8, 4), (16, 4), (32, 4), (128, 2),
         (256, 2), (256, 4), (512, 2), (512, 4), (1024, 1), (1024, 2),
         (1024, 4))
WIDTH = {"f32": 4, "bf16": 8, "f16": 8}
BITS = {"f32": torch.int32, "bf16": torch.int16, "f16": torch.int16}

CASES = [(op, dtype, g, vpt)
         for op in ("plain", "tail", "add_norm")
         for dtype in ("f32", "bf16", "f16")
         for g, vpt in TILES]
MULTI_CASES = [(dtype, g, vpt) for dtype in ("f32", "bf16", "f16")
               for g, vpt in TILES]


def _rows_per_block(g):
    return 256 // g if g < 128 else 1


def _pieces(rpb):
    """Row ranges: 16 workgroups, 7 rows, 1 row, the rest (all early)."""
    a = EARLY_BLOCKS * rpb
    return ((0, a), (a, a + 7), (a + 7, a + 8), (a + 8, 26 * rpb))


def _gain(rng, n, dtype):
    return gen.to_storage((1.0 + 0.1 * rng.standard_normal(n))
                          .astype(np.float32), dtype)


def _rows(rng, rows, n, dtype, scale=1.0):
    return gen.to_storage((scale * rng.standard_normal((rows, n)))
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


def _same_bits(a, b, dtype):
    return torch.equal(a.view(BITS[dtype]), b.view(BITS[dtype]))


@pytest.mark.parametrize("case", CASES,
                         ids=["-".join(map(str, c)) for c in CASES])
def test_early_and_late_gains_agree(oracle, case):
    op, dtype, g, vpt = case
    rpb = _rows_per_block(g)
    rows = 26 * rpb
    n = g * vpt * WIDTH[dtype] - 3        # the tile's last vector ragged
    label = f"early-gains {op} {dtype} rowtile {g}x{vpt} n={n} rows={rows}"
    say(label)
    rng = gen.rng_for(60000 + 31 * g + vpt + 7 * n)
    if op == "plain":
        inp = {"x": _rows(rng, rows, n, dtype),
               "gamma": _gain(rng, n, dtype), "eps": 1e-5, "dtype": dtype}
        ins = [dev(inp["x"], dtype)]
        eps = (inp["eps"],)
        keys = ("gamma",)
    elif op == "tail":
        inp = {"a": _rows(rng, rows, n, dtype),
               "r": _rows(rng, rows, n, dtype, 3.0),
               "gamma_post": _gain(rng, n, dtype),
               "gamma_pre": _gain(rng, n, dtype), "eps_post": 1e-8,
               "eps_pre": 1e-5, "dtype": dtype}
        ins = [dev(inp["a"], dtype), dev(inp["r"], dtype)]
        eps = (inp["eps_post"], inp["eps_pre"])
        keys = ("gamma_post", "gamma_pre")
    else:
        inp = {"a": _rows(rng, rows, n, dtype),
               "b": _rows(rng, rows, n, dtype, 0.5),
               "gamma": _gain(rng, n, dtype), "eps": 1e-5, "dtype": dtype}
        ins = [dev(inp["a"], dtype), dev(inp["b"], dtype)]
        eps = (inp["eps"],)
        keys = ("gamma",)
    ins += [dev(inp[k], dtype) for k in keys]
    outs_n = 1 if op == "plain" else 2
    whole = [torch.full_like(ins[0], float("nan")) for _ in range(outs_n)]
    parts = [torch.full_like(ins[0], float("nan")) for _ in range(outs_n)]
    pieces = _pieces(rpb)
    with snr.forced_shape("rowtile", g, vpt):
        _call(op, ins, whole, 0, rows, eps)
        assert snr.last_shape() == f"rowtile:{g}:{vpt}:{WIDTH[dtype]}", \
            snr.last_shape()
        for lo, hi in pieces:
            _call(op, ins, parts, lo, hi, eps)
    torch.cuda.synchronize()
    for w, p in zip(whole, parts):
        assert _same_bits(w, p, dtype), label

    # the first slice against the oracle
    lo, hi = pieces[0]
    sub = {k: (v[lo:hi] if isinstance(v, np.ndarray) and v.ndim == 2 else v)
           for k, v in inp.items()}
    got = [host_f64(p[lo:hi]) for p in parts]
    if op == "plain":
        check_plain(oracle, sub, got[0], label)
    elif op == "tail":
        check_tail(oracle, sub, got[0], got[1], label)
    else:
        check_add_norm(oracle, sub, got[0], got[1], label)


@pytest.mark.parametrize("case", MULTI_CASES,
                         ids=["-".join(map(str, c)) for c in MULTI_CASES])
def test_multi_early_and_late_gains_agree(oracle, case):
    dtype, g, vpt = case
    rpb = _rows_per_block(g)
    rows = 26 * rpb                        # two segments: 52 workgroups
    few = 8 * rpb                          # 8 + 8 = 16 workgroups
    n = g * vpt * WIDTH[dtype] - 3
    label = f"early-gains multi {dtype} rowtile {g}x{vpt} n={n}"
    say(label)
    rng = gen.rng_for(61000 + 31 * g + vpt + 7 * n)
    xs = [_rows(rng, rows, n, dtype, s) for s in (1.0, 4.0)]
    gs = [_gain(rng, n, dtype) for _ in range(2)]
    epss = (1e-5, 1e-6)
    dx = [dev(x, dtype) for x in xs]
    dg = [dev(gm, dtype) for gm in gs]
    whole = [torch.full_like(x, float("nan")) for x in dx]
    part = [torch.full_like(x[:few], float("nan")) for x in dx]
    with snr.forced_shape("rowtile", g, vpt):
        snr.rmsnorm_fwd_multi(list(zip(dx, dg, epss)), whole)
        assert snr.last_shape().startswith(f"multi:{g}:{vpt}:"), \
            snr.last_shape()
        snr.rmsnorm_fwd_multi([(x[:few], gm, e)
                               for x, gm, e in zip(dx, dg, epss)], part)
    torch.cuda.synchronize()
    for s in range(2):
        assert _same_bits(whole[s][:few], part[s], dtype), (label, s)
        inp = {"x": xs[s][:few], "gamma": gs[s], "eps": epss[s],
               "dtype": dtype}
        check_plain(oracle, inp, host_f64(part[s]), f"{label}-seg{s}")


@pytest.mark.parametrize("case", [("tail", 1, 6656, "rowtile:512:4:4"),
                                  ("tail", 16, 8192, "rowtile:512:4:4"),
                                  ("tail", 17, 6656, "rowtile:1024:2:4"),
                                  ("plain", 8, 4608, "rowtile:512:4:4"),
                                  ("norm_add", 2, 6656, "rowtile:512:4:4"),
                                  ("add_norm", 1, 6656, "rowtile:1024:2:4")],
                         ids=lambda c: "{}-rows{}-n{}".format(*c[:3]))
def test_decode_tile_choice(oracle, case):
    """f32 launches of at most 16 rows that would take the 1024 x 2 tile
    take 512 x 4 instead, except add_then_norm; the result matches the
    oracle. (The two tiles sum each row's squares in different orders, so
    their last bits may differ.)"""
    op, rows, n, want = case
    label = f"decode-tile {op} rows={rows} n={n}"
    say(label)
    rng = gen.rng_for(62000 + rows + n)
    if op == "plain":
        inp = {"x": _rows(rng, rows, n, "f32"), "gamma": _gain(rng, n, "f32"),
               "eps": 1e-5, "dtype": "f32"}
        run = lambda: [run_plain(inp)[0]]
    elif op == "tail":
        inp = {"a": _rows(rng, rows, n, "f32"),
               "r": _rows(rng, rows, n, "f32", 3.0),
               "gamma_post": _gain(rng, n, "f32"),
               "gamma_pre": _gain(rng, n, "f32"), "eps_post": 1e-8,
               "eps_pre": 1e-5, "dtype": "f32"}
        run = lambda: list(run_tail(inp))
    elif op == "norm_add":
        inp = {"a": _rows(rng, rows, n, "f32"),
               "b": _rows(rng, rows, n, "f32", 2.0),
               "gamma": _gain(rng, n, "f32"), "eps": 1e-8, "dtype": "f32"}
        run = lambda: [run_norm_add(inp)]
    else:
        inp = {"a": _rows(rng, rows, n, "f32"),
               "b": _rows(rng, rows, n, "f32", 0.5),
               "gamma": _gain(rng, n, "f32"), "eps": 1e-5, "dtype": "f32"}
        run = lambda: list(run_add_norm(inp))
    got = run()
    assert snr.last_shape() == want, (label, snr.last_shape())
    if op == "plain":
        check_plain(oracle, inp, got[0], label)
    elif op == "tail":
        check_tail(oracle, inp, got[0], got[1], label)
    elif op == "norm_add":
        check_norm_add(oracle, inp, got[0], None, label)
    else:
        check_add_norm(oracle, inp, got[0], got[1], label)
