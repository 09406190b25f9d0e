"""Seeded random sweeps, each case through the automatic dispatch and
checked against the oracle: 160 cases over every operation (plain norm,
tail, its two halves, several segments, Q8_1), every storage type, row
widths log-uniform from 1 to 70,000 (multiples of 32 for Q8_1) and 1-40
rows; and 40 cases with epsilon log-uniform from the smallest f32 subnormal
to 1e3. A case's draw depends only on its index, so a failure names its
inputs."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import (check_add_norm, check_norm_add, check_plain,  # noqa: E402
                         check_q8, check_tail, dev, host_f64, run_add_norm,
                         run_norm_add, run_plain, run_q8, run_tail, say)
from parity import NORMAL_MIN, TOLS, plain_error  # noqa: E402

pytestmark = pytest.mark.gpu

OPS = ["plain", "tail", "norm_add", "add_norm", "multi", "q8"]
CASES = 160


def draw(index):
    rng = np.random.default_rng(90000 + index)
    op = OPS[index % len(OPS)]
    st = ["f32", "bf16", "f16"][int(rng.integers(0, 3))]
    n = int(round(10 ** rng.uniform(0, np.log10(70000))))
    if op == "q8":
        n = max(32, n // 32 * 32)
    rows = int(rng.integers(1, 41))
    seed = int(rng.integers(0, 2 ** 31))
    return op, st, n, rows, seed


@pytest.mark.parametrize("index", range(CASES))
def test_random_case(oracle, index):
    op, st, n, rows, seed = draw(index)
    label = f"random#{index} {op} {st} rows={rows} n={n} seed={seed}"
    say(label)
    if op == "plain":
        inp = gen.random_plain(rows, n, seed, dtype=st)
        got, _ = run_plain(inp)
        check_plain(oracle, inp, got, label)
    elif op == "tail":
        inp = gen.random_tail(rows, n, seed, dtype=st)
        h, y = run_tail(inp, in_place=bool(seed & 1))
        check_tail(oracle, inp, h, y, label)
    elif op == "norm_add":
        inp = gen.random_pair("norm_add", rows, n, seed, dtype=st)
        scale = None if seed & 1 else 0.5
        out = run_norm_add(inp, scale=scale)
        check_norm_add(oracle, inp, out, scale, label)
    elif op == "add_norm":
        inp = gen.random_pair("add_norm", rows, n, seed, dtype=st)
        s, y = run_add_norm(inp)
        check_add_norm(oracle, inp, s, y, label)
    elif op == "q8":
        inp = gen.random_plain(rows, n, seed, dtype=st)
        check_q8(oracle, inp, run_q8(inp), label)
    else:
        # two to four segments of one width, own gains and epsilons
        k = 2 + seed % 3
        probs, inputs = [], []
        for j in range(k):
            inp = gen.random_plain(1 + (seed >> j) % rows, n, seed + j,
                                   dtype=st)
            inp["eps"] = [1e-5, 1e-6, 1e-3, 1e-8][j]
            inputs.append(inp)
            probs.append((dev(inp["x"], st), dev(inp["gamma"], st),
                          inp["eps"]))
        outs = snr.rmsnorm_fwd_multi(probs)
        torch.cuda.synchronize()
        for inp, out in zip(inputs, outs):
            from gpu_helpers import f32
            want = oracle.rmsnorm(f32(inp, "x"), f32(inp, "gamma"),
                                  inp["eps"])
            err = plain_error(host_f64(out), want, NORMAL_MIN[st])
            assert err <= TOLS[st], (label, err)
        say(f"{label}: {k} segments ok ({snr.last_shape()})")


# ---------------------------------------------------------------------------
# Epsilon sweep: every operation with epsilon log-uniform from the smallest
# f32 subnormal (2^-149) to 1e3, so that the mean square is negligible, comparable
# to epsilon, or dominated by it. Draws of their own (the cases above keep
# theirs).
# ---------------------------------------------------------------------------
EPS_CASES = 40
EPS_LOG_LO = np.log10(2.0 ** -149)


def draw_eps(index):
    rng = np.random.default_rng(95000 + index)
    op = ["plain", "tail", "norm_add", "add_norm", "q8"][index % 5]
    st = ["f32", "bf16", "f16"][int(rng.integers(0, 3))]
    n = int(round(10 ** rng.uniform(0, np.log10(20000))))
    if op == "q8":
        n = max(32, n // 32 * 32)
    rows = int(rng.integers(1, 21))
    seed = int(rng.integers(0, 2 ** 31))
    eps = [float(np.float32(10 ** rng.uniform(EPS_LOG_LO, 3.0)))
           for _ in range(2)]
    return op, st, n, rows, seed, eps


@pytest.mark.parametrize("index", range(EPS_CASES))
def test_random_epsilon(oracle, index):
    op, st, n, rows, seed, eps = draw_eps(index)
    label = (f"random-eps#{index} {op} {st} rows={rows} n={n} seed={seed} "
             f"eps={eps[0]:.3g},{eps[1]:.3g}")
    say(label)
    assert all(e > 0 for e in eps)
    if op == "plain":
        inp = gen.random_plain(rows, n, seed, dtype=st)
        inp["eps"] = eps[0]
        got, _ = run_plain(inp)
        check_plain(oracle, inp, got, label)
    elif op == "tail":
        inp = gen.random_tail(rows, n, seed, dtype=st)
        inp["eps_post"], inp["eps_pre"] = eps
        h, y = run_tail(inp)
        check_tail(oracle, inp, h, y, label)
    elif op == "norm_add":
        inp = gen.random_pair("norm_add", rows, n, seed, dtype=st)
        inp["eps"] = eps[0]
        out = run_norm_add(inp)
        check_norm_add(oracle, inp, out, None, label)
    elif op == "add_norm":
        inp = gen.random_pair("add_norm", rows, n, seed, dtype=st)
        inp["eps"] = eps[0]
        s, y = run_add_norm(inp)
        check_add_norm(oracle, inp, s, y, label)
    else:
        inp = gen.random_plain(rows, n, seed, dtype=st)
        inp["eps"] = eps[0]
        check_q8(oracle, inp, run_q8(inp), label)
