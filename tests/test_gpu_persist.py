"""The persistent row tiles (forced shape "persist") against the oracle, and
bit for bit against the row-tile kernel with the same lanes per row and
loads per lane (the arithmetic is shared; only the way rows reach the
registers differs). Large row counts give every workgroup many trips
through its pipelined loop (odd and even counts)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import (check_add_norm, check_norm_add, check_plain,  # noqa: E402
                         check_tail, run_add_norm, run_norm_add, run_plain,
                         run_tail, say)

pytestmark = pytest.mark.gpu

VEC = {"f32": 4, "bf16": 8, "f16": 8}
SHAPES = [(128, 2), (256, 2), (512, 2), (1024, 1), (1024, 2)]
OPS = ["plain", "tail", "norm_add", "add_norm"]


def _inputs(op, st, rows, n, seed):
    if op == "plain":
        return gen.random_plain(rows, n, seed, dtype=st)
    if op == "tail":
        return gen.random_tail(rows, n, seed, dtype=st)
    return gen.random_pair(op, rows, n, seed, dtype=st)


def _run(op, inp):
    if op == "plain":
        return [run_plain(inp)[0]]
    if op == "tail":
        return list(run_tail(inp))
    if op == "norm_add":
        return [run_norm_add(inp, scale=1.25)]
    return list(run_add_norm(inp))


def _check(oracle, op, inp, outs, label):
    if op == "plain":
        check_plain(oracle, inp, outs[0], label)
    elif op == "tail":
        check_tail(oracle, inp, outs[0], outs[1], label)
    elif op == "norm_add":
        check_norm_add(oracle, inp, outs[0], 1.25, label)
    else:
        check_add_norm(oracle, inp, outs[0], outs[1], label)


def _cases():
    # 1024 x 4 is compiled for the plain norm only
    return ([(op, st, g, v) for op in OPS for st in ("f32", "bf16", "f16")
             for g, v in SHAPES] +
            [("plain", st, 1024, 4) for st in ("f32", "bf16", "f16")])


@pytest.mark.parametrize("case", _cases(),
                         ids=lambda c: "{}-{}-g{}-v{}".format(*c))
def test_persist_matches_oracle_and_rowtile(oracle, case):
    op, st, g, v = case
    w = VEC[st]
    nv = g * v - g // 2          # a partly filled tile
    n = nv * w
    rows = 700
    label = f"persist-{op}-{st}-g{g}-v{v}-n{n}"
    say(f"{label} rows={rows}")
    inp = _inputs(op, st, rows, n, 32000 + g + v + n)
    with snr.forced_shape("persist", g, v):
        got = _run(op, inp)
        assert snr.last_shape() == f"persist:{g}:{v}:{w}", snr.last_shape()
    _check(oracle, op, inp, got, label)
    with snr.forced_shape("rowtile", g, v):
        ref = _run(op, inp)
    for a, b in zip(got, ref):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), label


@pytest.mark.parametrize("case", [("tail", "f32", 1024, 2, 4099),
                                  ("tail", "bf16", 512, 2, 4096),
                                  ("plain", "f16", 1024, 1, 8195),
                                  ("add_norm", "bf16", 128, 2, 20001)],
                         ids=lambda c: "{}-{}-g{}-v{}-rows{}".format(*c))
def test_persist_many_trips(oracle, case):
    """Thousands of rows: each workgroup of the resident grid takes several
    rows in turn. Bit-equal to the row tile; sampled rows against the
    oracle."""
    op, st, g, v, rows = case
    w = VEC[st]
    n = (g * v - 8) * w
    label = f"persist-trips-{op}-{st}-g{g}-v{v}-rows{rows}"
    say(label)
    inp = _inputs(op, st, rows, n, 33000 + rows)
    with snr.forced_shape("persist", g, v):
        got = _run(op, inp)
    with snr.forced_shape("rowtile", g, v):
        ref = _run(op, inp)
    for a, b in zip(got, ref):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), label
    pick = np.r_[0:3, rows // 2:rows // 2 + 3, rows - 3:rows]
    sub = {k: (val[pick] if isinstance(val, np.ndarray) and val.ndim == 2
               else val) for k, val in inp.items()}
    _check(oracle, op, sub, [o[pick] for o in got], label + "-sampled")


def test_persist_rejects_ragged_rows():
    inp = gen.random_plain(4, 4 * 100 + 1, 34000)
    with snr.forced_shape("persist", 128, 2):
        with pytest.raises(snr.SnrError):
            run_plain(inp)


@pytest.mark.parametrize("case", [("bf16", 16384, 256, "persist:1024:2:8"),
                                  ("f16", 12288, 1000, "persist:1024:2:8"),
                                  ("bf16", 16384, 255, "rowtile:1024:2:8"),
                                  ("bf16", 16379, 300, "rowtile:1024:2:8"),
                                  ("bf16", 6656, 4096, "rowtile:512:2:8"),
                                  ("bf16", 24576, 256, "persist:1024:4:8"),
                                  ("f32", 16384, 1024, "persist:1024:4:4"),
                                  ("f32", 12288, 1023, "rowtile:1024:4:4"),
                                  ("f32", 16381, 2048, "rowtile:1024:4:4"),
                                  ("f32", 8192, 1024, "persist:1024:2:4"),
                                  ("f32", 8184, 1024, "rowtile:1024:2:4"),
                                  ("f32", 6656, 4096, "rowtile:1024:2:4")],
                         ids=lambda c: "{}-n{}-rows{}".format(*c[:3]))
def test_automatic_plain_persist_choice(oracle, case):
    """The plain norm takes the persistent tile automatically only with 1024
    lanes per row and rows without a ragged end: in 16-bit storage over 256
    rows or more, in f32 over 1024 rows or more at four loads per lane or
    with a row that fills a two-load tile (n = 8192). The
    result is bit-equal to the forced row tile and matches the oracle on
    sampled rows."""
    st, n, rows, want = case
    label = f"auto-plain-{st}-n{n}-rows{rows}"
    say(label)
    inp = _inputs("plain", st, rows, n, 35000 + rows + n)
    got = _run("plain", inp)
    assert snr.last_shape() == want, (label, snr.last_shape())
    _, g, v, _w = want.split(":")
    with snr.forced_shape("rowtile", int(g), int(v)):
        ref = _run("plain", inp)
    assert np.array_equal(got[0].view(np.uint8), ref[0].view(np.uint8)), label
    pick = np.r_[0:3, rows // 2:rows // 2 + 3, rows - 3:rows]
    sub = {k: (val[pick] if isinstance(val, np.ndarray) and val.ndim == 2
               else val) for k, val in inp.items()}
    _check(oracle, "plain", sub, [got[0][pick]], label + "-sampled")


@pytest.mark.parametrize("case", [("tail", "bf16", 6656, 1024, "rowtile:512:2:8"),
                                  ("tail", "bf16", 6656, 1100, "persist:512:2:8"),
                                  ("tail", "bf16", 6656, 512, "persist:512:2:8"),
                                  ("norm_add", "f16", 6656, 1000, "rowtile:512:2:8"),
                                  ("tail", "bf16", 16384, 300, "rowtile:1024:2:8"),
                                  ("tail", "bf16", 12288, 1, "rowtile:1024:2:8"),
                                  ("add_norm", "f16", 12288, 16, "rowtile:1024:2:8"),
                                  ("tail", "bf16", 12288, 17, "persist:1024:2:8"),
                                  ("plain", "f16", 12288, 300, "rowtile:1024:2:8")],
                         ids=lambda c: "{}-{}-n{}-rows{}".format(*c[:4]))
def test_automatic_choice_one_round(oracle, case):
    """Where the row tile holds every row at once on this GPU and the
    persistent grid (a larger register tile, so fewer resident workgroups)
    would not, the row tile is kept: on MI355X the 16-bit tail at 512 x 2
    holds 1024 rows in one round of row tiles against 512 persistent
    workgroups. So is it for launches of at most 16 rows at 1024 lanes. Results bit-equal to the forced row tile; sampled rows
    against the oracle. Also a regression test: resident counts were once
    cached per kernel signature, so the first persistent kernel of a process
    fixed the count for all of them."""
    op, st, n, rows, want = case
    label = f"auto-round-{op}-{st}-n{n}-rows{rows}"
    say(label)
    # a persistent kernel that holds fewer workgroups (256) runs first: the
    # resident counts are kept per kernel, so it must not move the choice
    warm = gen.random_plain(8, 1024 * 4 * 4, 36999)
    with snr.forced_shape("persist", 1024, 4):
        run_plain(warm)
    inp = _inputs(op, st, rows, n, 36000 + rows + n)
    got = _run(op, inp)
    assert snr.last_shape() == want, (label, snr.last_shape())
    _, g, v, _w = want.split(":")
    with snr.forced_shape("rowtile", int(g), int(v)):
        ref = _run(op, inp)
    for a, b in zip(got, ref):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), label
    pick = np.unique(np.clip(np.r_[0:3, rows // 2:rows // 2 + 3,
                                   rows - 3:rows], 0, rows - 1))
    sub = {k: (val[pick] if isinstance(val, np.ndarray) and val.ndim == 2
               else val) for k, val in inp.items()}
    _check(oracle, op, sub, [o[pick] for o in got], label + "-sampled")


@pytest.mark.parametrize("cap,rows", [(3, 22), (4, 21)])
@pytest.mark.parametrize("case", _cases(),
                         ids=lambda c: "{}-{}-g{}-v{}".format(*c))
def test_persist_walks_many_rows(oracle, case, cap, rows):
    """The persistent grid capped at a few workgroups (snr_force_grid), so
    each walks 5 to 8 rows through its two row buffers (odd and even trip
    counts, the peeled first row and the unrolled loop's tail): the same
    bits as the row tile and the oracle's values."""
    op, st, g, v = case
    w = VEC[st]
    nv = g * v - g // 2
    n = nv * w
    label = f"persist-walk-{op}-{st}-g{g}-v{v}-cap{cap}-r{rows}"
    say(label)
    inp = _inputs(op, st, rows, n, 33000 + g + v + n + cap)
    with snr.forced_shape("persist", g, v), snr.forced_grid(cap):
        got = _run(op, inp)
        assert snr.last_shape() == f"persist:{g}:{v}:{w}", snr.last_shape()
    _check(oracle, op, inp, got, label)
    with snr.forced_shape("rowtile", g, v):
        ref = _run(op, inp)
    for a, b in zip(got, ref):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), label
