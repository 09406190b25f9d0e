"""GPU parity of the tail in 16-bit storage, the in-place tail, and the tail's
two halves (norm_then_add, add_then_norm) against the f64 oracle.

Every (operation, storage) pair runs every compiled dispatch shape (forced)
on a ragged row, the full-size workloads run with the automatic choice, and
the in-place and scaled forms are checked.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import (check_add_norm, check_norm_add,  # noqa: E402
                         check_plain, check_tail, f32, run_add_norm,
                         run_norm_add, run_plain, run_tail, say)
from parity import NORMAL_MIN, scaled_error  # noqa: E402

pytestmark = pytest.mark.gpu

VEC = {"f32": 4, "bf16": 8, "f16": 8}
# row-tile shapes the automatic choice can reach (compiled for every pair)
AUTO_ROWTILE = [(1, 4), (2, 4), (4, 4), (8, 4), (16, 4), (32, 4), (128, 2),
                (128, 8), (256, 2), (256, 4), (512, 2), (512, 4), (1024, 1),
                (1024, 2), (1024, 4), (1024, 8)]
PAIRS = [("tail", "bf16"), ("tail", "f16"), ("plain", "f16"),
         ("norm_add", "f32"), ("norm_add", "bf16"), ("norm_add", "f16"),
         ("add_norm", "f32"), ("add_norm", "bf16"), ("add_norm", "f16")]
WIDE16 = {("norm_add", "f32"), ("add_norm", "f32")}


def make_inputs(op, st, rows, n, seed):
    if op == "plain":
        return gen.random_plain(rows, n, seed, dtype=st)
    if op == "tail":
        return gen.random_tail(rows, n, seed, dtype=st)
    return gen.random_pair(op, rows, n, seed, dtype=st)


def run_and_check(oracle, op, inp, label, scale=None):
    if op == "plain":
        got, _ = run_plain(inp)
        check_plain(oracle, inp, got, label)
    elif op == "tail":
        h, y = run_tail(inp)
        check_tail(oracle, inp, h, y, label)
    elif op == "norm_add":
        out = run_norm_add(inp, scale=scale)
        check_norm_add(oracle, inp, out, scale, label)
    else:
        s, y = run_add_norm(inp)
        check_add_norm(oracle, inp, s, y, label)
    return snr.last_shape()


def _forced_cases():
    cases = []
    for op, st in PAIRS:
        shapes = [("rowtile", g, v) for g, v in AUTO_ROWTILE]
        if (op, st) in WIDE16:
            shapes.append(("rowtile", 1024, 16))
        shapes += [("split", 0, 8), ("multipass", 0, 8)]
        for kind, g, v in shapes:
            cases.append((op, st, kind, g, v))
    return cases


@pytest.mark.parametrize("case", _forced_cases(),
                         ids=lambda c: "{}-{}-{}-g{}-v{}".format(*c))
def test_forced_shape(oracle, case):
    """Every compiled shape of the pair, on rows ragged by the largest
    remainder (W - 1 elements past the last whole vector)."""
    op, st, kind, g, v = case
    w = VEC[st]
    if kind == "rowtile":
        nv = max(1, g * v - g // 2 - (1 if g == 1 else 0))
    elif kind == "split":
        nv = 2 * (4096 // w) + 5   # three chunks of 4096 elements
    else:
        nv = 2 * 4096 + 5          # three chunks of 256 x 16 vectors
    n = nv * w + w - 1
    rows = 19
    label = f"{op}-{st}-{kind}-g{g}-v{v}-n{n}"
    say(f"forced {label} rows={rows}")
    inp = make_inputs(op, st, rows, n, 20000 + g * 7 + v + n)
    with snr.forced_shape(kind, g, v):
        shape = run_and_check(oracle, op, inp, label,
                              scale=1.5 if op == "norm_add" else None)
    if kind == "rowtile":
        assert shape == f"rowtile:{g}:{v}:{w}", shape
    elif kind == "split":
        assert shape == f"split:256:{4096 // (256 * w)}:{w}:3", shape
    else:
        assert shape == f"multipass:256:16:{w}:3", shape


SPLIT_PAIRS = PAIRS + [("plain", "f32"), ("plain", "bf16"), ("tail", "f32")]


@pytest.mark.parametrize("groups,rows,chunks", [(2, 19, 3), (3, 20, 1),
                                                (5, 23, 2)])
@pytest.mark.parametrize("op_st", SPLIT_PAIRS, ids=lambda p: "-".join(p))
def test_forced_split_walks_many_rows(oracle, op_st, groups, rows, chunks):
    """The split-row kernel with its rows in flight capped (snr_force_grid),
    so every workgroup walks 4 to 10 rows: each register ring (the
    four row buffers, the second stream's, and the 16-bit tail's f32 h) is
    reused several times, with uneven trip counts, on ragged rows. Every
    output matches the oracle and no wait gives up."""
    op, st = op_st
    w = VEC[st]
    nv = (chunks - 1) * (4096 // w) + 5
    n = nv * w + w - 1
    label = f"split-walk-{op}-{st}-g{groups}-r{rows}-n{n}"
    say(f"{label}")
    inp = make_inputs(op, st, rows, n, 30000 + groups * 101 + rows + n)
    with snr.forced_shape("split", 0, 8), snr.forced_grid(groups):
        shape = run_and_check(oracle, op, inp, label,
                              scale=0.75 if op == "norm_add" else None)
    assert shape == f"split:256:{4096 // (256 * w)}:{w}:{chunks}", shape
    assert snr.split_timeouts() == 0


@pytest.mark.parametrize("name", ["tail_4096x6656_bf16", "tail_4096x6656_f16",
                                  "norm_add_4096x6656_f32",
                                  "add_norm_4096x6656_f32"])
def test_workload_full_size(oracle, name):
    cfg = gen.CONFIGS[name]
    say(f"workload {name}")
    inp = gen.make(cfg)
    run_and_check(oracle, cfg.kind, inp, name)


@pytest.mark.parametrize("op_st", PAIRS + [("tail", "f32")])
@pytest.mark.parametrize("n", [1, 2, 3, 7, 9, 100, 6657, 65536 + 5])
def test_ragged_auto(oracle, op_st, n):
    op, st = op_st
    rows = 13
    say(f"ragged {op} {st} n={n}")
    inp = make_inputs(op, st, rows, n, 21000 + n)
    run_and_check(oracle, op, inp, f"ragged-{op}-{st}-{n}")


@pytest.mark.parametrize("st", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [3, 6656, 65536])
def test_tail_inplace(oracle, st, n):
    """sandwich_tail_inplace updates the residual and returns y."""
    rows = 11
    say(f"tail in place {st} n={n}")
    inp = gen.random_tail(rows, n, 22000 + n, dtype=st)
    h, y = run_tail(inp, in_place=True)
    check_tail(oracle, inp, h, y, f"tail-inplace-{st}-{n}")


@pytest.mark.parametrize("st", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("scale", [None, 2.5, -0.75])
def test_norm_add_scale_and_in_place(oracle, st, scale):
    rows, n = 33, 4099
    say(f"norm_add {st} scale={scale}")
    inp = gen.random_pair("norm_add", rows, n, 23000, dtype=st)
    out = run_norm_add(inp, scale=scale)
    check_norm_add(oracle, inp, out, scale, f"norm-add-{st}-{scale}")
    out_ip = run_norm_add(inp, scale=scale, in_place=True)
    check_norm_add(oracle, inp, out_ip, scale, f"norm-add-inplace-{st}")
    assert np.array_equal(out, out_ip)


@pytest.mark.parametrize("st", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("into", ["a", "b"])
def test_add_norm_in_place(oracle, st, into):
    rows, n = 21, 2051
    say(f"add_norm in place {st} into {into}")
    inp = gen.random_pair("add_norm", rows, n, 24000, dtype=st)
    s, y = run_add_norm(inp, sum_into=into)
    check_add_norm(oracle, inp, s, y, f"add-norm-into-{into}-{st}")
    s2, y2 = run_add_norm(inp)
    assert np.array_equal(s, s2) and np.array_equal(y, y2)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n", [256, 6656])
@pytest.mark.parametrize("op", ["tail", "add_norm"])
def test_second_norm_reads_the_f32_intermediate(oracle, op, n, dtype):
    """The tail's h and add_then_norm's sum are stored rounded, and the
    second norm works from their f32 values. On rows where normalising the
    rounded copy would put y past the bf16 gate (tests/spikes.py; shown on
    the CPU by test_intermediate_rounding_cpu.py), y stays within one unit
    roundoff of the exact result, and so does the stored intermediate."""
    from parity import tail_errors
    from spikes import SIGNIFICAND_BITS, add_norm_spikes, tail_spikes
    say(f"second norm from f32 intermediate: {op} n={n} {dtype}")
    bound = 2.0 ** -SIGNIFICAND_BITS[dtype] * 1.001 + 1e-6
    fl = NORMAL_MIN[dtype]
    if op == "tail":
        inp = tail_spikes(16, n, 33000 + n, dtype)
        h, y = run_tail(inp)
        r, gq = f32(inp, "r"), f32(inp, "gamma_pre")
        o = oracle.sandwich_tail(f32(inp, "a"), r, f32(inp, "gamma_post"),
                                 inp["eps_post"], gq, inp["eps_pre"])
        e_inter, ey = tail_errors(h, y, o, r, gq, fl)
    else:
        inp = add_norm_spikes(16, n, 34000 + n, dtype)
        s, y = run_add_norm(inp)
        a, b, g = f32(inp, "a"), f32(inp, "b"), f32(inp, "gamma")
        ws, wy, d = oracle.add_then_norm(a, b, g, inp["eps"])
        den = np.abs(a.astype(np.float64)) + np.abs(b)
        e_inter = scaled_error(s, ws, den, fl)[0]
        ey = scaled_error(y, wy, np.abs(g.astype(np.float64)) * den /
                          d[:, None], fl)[0]
    say(f"  intermediate err {e_inter:.3e}, y err {ey:.3e} (bound {bound:.3e}) "
        f"shape {snr.last_shape()}")
    assert e_inter <= bound and ey <= bound, (e_inter, ey)


@pytest.mark.parametrize("op", ["tail", "add_norm"])
def test_multipass_second_norm_bound(oracle, op):
    """The multi-pass kernels re-read the stored intermediate for the last
    pass, with the mean of squares of its f32 values: y carries at most two
    bf16 roundings on the same rows, inside the 8e-3 gate."""
    from parity import tail_errors
    from spikes import add_norm_spikes, tail_spikes
    say(f"multipass second norm: {op}")
    bound = 2.0 * 2.0 ** -8 * 1.001 + 1e-6
    fl = NORMAL_MIN["bf16"]
    with snr.forced_shape("multipass", 0, 8):
        if op == "tail":
            inp = tail_spikes(8, 6656, 35000, "bf16")
            h, y = run_tail(inp)
            shape = snr.last_shape()
            r, gq = f32(inp, "r"), f32(inp, "gamma_pre")
            o = oracle.sandwich_tail(f32(inp, "a"), r, f32(inp, "gamma_post"),
                                     inp["eps_post"], gq, inp["eps_pre"])
            e_inter, ey = tail_errors(h, y, o, r, gq, fl)
        else:
            inp = add_norm_spikes(8, 6656, 36000, "bf16")
            s, y = run_add_norm(inp)
            shape = snr.last_shape()
            a, b, g = f32(inp, "a"), f32(inp, "b"), f32(inp, "gamma")
            ws, wy, d = oracle.add_then_norm(a, b, g, inp["eps"])
            den = np.abs(a.astype(np.float64)) + np.abs(b)
            e_inter = scaled_error(s, ws, den, fl)[0]
            ey = scaled_error(y, wy, np.abs(g.astype(np.float64)) * den /
                              d[:, None], fl)[0]
    assert shape.startswith("multipass:"), shape
    say(f"  intermediate err {e_inter:.3e}, y err {ey:.3e} (bound {bound:.3e})")
    assert e_inter <= 2.0 ** -8 * 1.001 + 1e-6 and ey <= bound, (e_inter, ey)


