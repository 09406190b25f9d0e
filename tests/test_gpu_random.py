"""Seeded random sweep: 160 cases drawn over every operation (plain norm,
tail, its two halves, several segments, Q8_1), every storage type, row
widths log-uniform from 1 to 70,000 (multiples of 32 for Q8_1) and 1-40
rows, each through the automatic dispatch and checked against the oracle.
A case's draw depends only on its index, so a failure names its inputs."""
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
