"""GPU parity of RMSNorm into Q8_1 records against the f64 oracle: every
compiled dispatch shape, the full-size workloads, ragged and edge rows, and
all three storage types."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import check_q8, dev, run_q8, say  # noqa: E402

pytestmark = pytest.mark.gpu

VEC = {"f32": 4, "bf16": 8, "f16": 8}
Q8_ROWTILE = [(8, 4), (16, 4), (32, 4), (128, 2), (128, 8), (256, 2),
              (256, 4), (512, 2), (512, 4), (1024, 1), (1024, 2), (1024, 4),
              (1024, 8)]


def _forced_cases():
    cases = []
    for st in ("f32", "bf16", "f16"):
        shapes = [("rowtile", g, v) for g, v in Q8_ROWTILE]
        if st == "f32":
            shapes.append(("rowtile", 1024, 16))
        else:
            shapes.append(("rowtile", 4, 4))
        shapes.append(("multipass", 0, 8))
        cases += [(st, k, g, v) for k, g, v in shapes]
    return cases


@pytest.mark.parametrize("case", _forced_cases(),
                         ids=lambda c: "{}-{}-g{}-v{}".format(*c))
def test_forced_shape(oracle, case):
    """Each compiled shape on rows that fill its tile only partly (the row's
    vector count is the largest whole number of 32-element blocks below
    g * vpt - g / 2)."""
    st, kind, g, v = case
    w = VEC[st]
    bv = 32 // w
    if kind == "rowtile":
        nv = max(bv, (g * v - g // 2) // bv * bv)
    else:
        nv = 2 * 4096 + 8          # three chunks of 256 x 16 vectors
    n = nv * w
    rows = 19
    label = f"q8-{st}-{kind}-g{g}-v{v}-n{n}"
    say(f"forced {label} rows={rows}")
    inp = gen.random_plain(rows, n, 26000 + g * 7 + v + n, dtype=st)
    with snr.forced_shape(kind, g, v):
        blocks = run_q8(inp)
        shape = snr.last_shape()
    check_q8(oracle, inp, blocks, label)
    if kind == "rowtile":
        assert shape == f"rowtile:{g}:{v}:{w}", shape
    else:
        assert shape == f"multipass:256:16:{w}:3", shape


def _persistent_cases():
    # the tiles holding at most 16 values per lane run persistent
    cases = []
    for st in ("f32", "bf16", "f16"):
        extra = [(1024, 16)] if st == "f32" else [(4, 4)]
        for g, v in Q8_ROWTILE + extra:
            if v * VEC[st] <= 16:
                cases.append((st, g, v))
    return cases


@pytest.mark.parametrize("case", _persistent_cases(),
                         ids=lambda c: "{}-g{}-v{}".format(*c))
def test_persistent_walks_many_rows(oracle, case):
    """The persistent Q8_1 tiles with their grid capped at three workgroups
    (snr_force_grid), so each walks 5 or 6 row blocks (its prefetch, the
    peeled first block and the loop's tail), the last block partly filled:
    records equal to the uncapped launch's, and the oracle's."""
    st, g, v = case
    w = VEC[st]
    bv = 32 // w
    nv = max(bv, (g * v - g // 2) // bv * bv)
    n = nv * w
    rpb = 256 // g if g < 128 else 1      # rows per workgroup
    rows = rpb * 16 + max(1, rpb // 2)    # 17 row blocks, the last partial
    label = f"q8-walk-{st}-g{g}-v{v}-n{n}-r{rows}"
    say(label)
    inp = gen.random_plain(rows, n, 27000 + g * 7 + v + n, dtype=st)
    with snr.forced_shape("rowtile", g, v), snr.forced_grid(3):
        blocks = run_q8(inp)
        shape = snr.last_shape()
    assert shape == f"rowtile:{g}:{v}:{w}", shape
    check_q8(oracle, inp, blocks, label)
    with snr.forced_shape("rowtile", g, v):
        ref = run_q8(inp)
    assert np.array_equal(np.asarray(blocks), np.asarray(ref)), label


@pytest.mark.parametrize("name", ["q8_4096x6656_f32", "q8_4096x6656_bf16",
                                  "q8_1x2560_f32", "q8_edge_256x6656_f32"])
def test_workload_full_size(oracle, name):
    cfg = gen.CONFIGS[name]
    say(f"workload {name}")
    inp = gen.make(cfg)
    _, near = check_q8(oracle, inp, run_q8(inp), name)
    # the tie band is a sliver: nearly every code is compared exactly
    assert near <= 1e-2 * cfg.rows * cfg.n


@pytest.mark.parametrize("st", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [32, 64, 96, 2560, 6656, 65536, 65536 + 32,
                               4 * 65536])
def test_widths_auto(oracle, st, n):
    """Automatic shape choice from one block up to rows the multi-pass
    kernels take."""
    rows = 13
    say(f"q8 auto {st} n={n}")
    inp = gen.random_plain(rows, n, 27000 + n, dtype=st)
    check_q8(oracle, inp, run_q8(inp), f"q8-auto-{st}-{n}")


def test_zero_rows_and_blocks(oracle):
    """An all-zero row, and zero blocks inside a row, encode as d = 0 and
    q = 0; the row's other blocks are unaffected."""
    rows, n = 4, 256
    inp = gen.random_plain(rows, n, 28000)
    inp["x"][0] = 0.0
    inp["x"][1, 32:96] = 0.0
    inp["x"][2, :] = 0.0
    inp["x"][2, 200] = -7.0
    blocks = run_q8(inp)
    check_q8(oracle, inp, blocks, "q8-zero-blocks")
    assert not blocks[0].any()
    assert not blocks[1, 1:3].any()
    assert not blocks[2, [0, 1, 2, 3, 4, 5, 7]].any()
    d, s, q = snr.q8_1_fields(torch.from_numpy(blocks))
    assert q[2, 6, 200 - 192].item() == -127


def test_rows_zero_and_out_argument(oracle):
    x = torch.empty((0, 64), device="cuda:0")
    g = torch.ones(64, device="cuda:0")
    assert snr.rmsnorm_q8_1(x, g, 1e-5).shape == (0, 2, 36)
    inp = gen.random_plain(5, 128, 29000)
    xs, gs = dev(inp["x"], "f32"), dev(inp["gamma"], "f32")
    out = torch.full((5, 4, 36), 0xAB, dtype=torch.uint8, device="cuda:0")
    r = snr.rmsnorm_q8_1(xs, gs, 1e-5, out=out)
    assert r is out
    check_q8(oracle, inp, out.cpu().numpy(), "q8-out-arg")
    with pytest.raises(ValueError):
        snr.rmsnorm_q8_1(xs[:, :100].contiguous(), gs[:100].contiguous(),
                         1e-5)


def test_tiny_blocks_and_subnormal_inputs(oracle):
    """Blocks whose scale d is an f32 subnormal (amax ~ 1e-37) and rows of
    subnormal inputs whose normalised values are normal: the quotient
    v / d must stay finite and accurate (no reciprocal of a subnormal)."""
    rng = gen.rng_for(28100)
    rows, n = 4, 256
    x = rng.standard_normal((rows, n)).astype(np.float32)
    x[0, 0:32] *= np.float32(1e-37)      # normalised block ~1e-37: d subnormal
    x[1, 64:96] *= np.float32(3e-36)
    x[2] *= np.float32(1e-40)            # subnormal inputs, eps dominates
    x[3, :] = 0.0
    x[3, 5] = np.float32(1e-44)          # one subnormal element
    g = (1.0 + 0.1 * rng.standard_normal(n)).astype(np.float32)
    inp = {"x": x, "gamma": g, "eps": 1e-5, "dtype": "f32"}
    blocks = run_q8(inp)
    check_q8(oracle, inp, blocks, "q8-tiny")
    d, s, q = snr.q8_1_fields(torch.from_numpy(blocks))
    assert int(q[0, 0].abs().max()) == 127      # the block's own scale


@pytest.mark.parametrize("st", ["f32", "bf16"])
def test_subnormal_epsilon(oracle, st):
    """epsilon = the smallest f32 subnormal (2^-149): a zero row still
    encodes d = 0 and q = 0 (1/rms stays finite), and rows whose mean square
    plus epsilon falls below the smallest normal match the oracle."""
    say(f"q8 subnormal epsilon {st}")
    rng = gen.rng_for(28200)
    rows, n = 5, 256
    x = rng.standard_normal((rows, n)).astype(np.float32)
    x[0] = 0.0
    x[1] = 0.0
    x[1, 37] = np.float32(1e-18)          # mean square 1e-36 / 256 < 2^-126
    x[2] *= np.float32(1e-20)             # squares near 1e-40 ... 1e-39
    x[2] = np.where(np.abs(x[2]) < 1e-20, np.float32(1e-20), x[2])
    x[3, 64:] = 0.0                       # zero blocks after normal ones
    g = (1.0 + 0.1 * rng.standard_normal(n)).astype(np.float32)
    eps = float(np.float32(2.0 ** -149))
    inp = {"x": gen.to_storage(x, st), "gamma": gen.to_storage(g, st),
           "eps": eps, "dtype": st}
    blocks = run_q8(inp)
    check_q8(oracle, inp, blocks, f"q8-subnormal-eps-{st}")
    assert not blocks[0].any()
    assert not blocks[3, 2:].any()


def test_exact_ties_round_to_even(oracle):
    """A block whose quotients x / d are exact ties (rms = 64 and d = 1/32
    exactly, t = x / 2): the codes are round-half-even of the exact
    quotient, equal to the oracle's with no tie band."""
    vals = [254, 1, 3, 5, 7, -1, -3, -5, -7, 200, 160, 28, 2] + [0] * 19
    x = np.array([vals, [-v for v in vals]], np.float32)
    inp = {"x": x, "gamma": np.ones(32, np.float32), "eps": 1e-30,
           "dtype": "f32"}
    blocks = run_q8(inp)
    d, s, q = snr.q8_1_fields(torch.from_numpy(blocks))
    want = [127, 0, 2, 2, 4, 0, -2, -2, -4, 100, 80, 14, 1] + [0] * 19
    assert q[0, 0].tolist() == want
    assert q[1, 0].tolist() == [-v for v in want]
    assert float(d[0, 0]) == 1.0 / 32.0 and float(d[1, 0]) == 1.0 / 32.0
    _, _, _, qo = oracle.rmsnorm_q8_1(x, inp["gamma"], inp["eps"])
    assert np.array_equal(q.reshape(2, 32).numpy(), qo)
