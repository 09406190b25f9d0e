"""GPU parity: the HIP kernels (through the C ABI) against the f64 oracle on
the same seeded inputs, element by element.

Covers every configuration at full size in the launch configuration the
benchmark times (automatic shape choice), every compiled dispatch shape forced
on rows it is not normally chosen for (ragged within its tile), the split-row
path with 1..5 chunks, ragged and misaligned rows, in-place operation,
sentinel prefill, determinism, rows = 0, and bf16 round-to-nearest-even.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import _lib  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import (DEV, check_plain, check_tail, dev,  # noqa: E402
                         host_f64, run_plain, run_tail, say)

pytestmark = pytest.mark.gpu

# Row-tile shapes compiled for every (operation, storage); 1024 x 16 exists
# only where the row fits the registers of a 1024-lane workgroup.
ROWTILE_SHAPES = [(1, 4), (2, 4), (4, 4), (8, 4), (16, 4), (32, 4),
                  (64, 2), (64, 4), (64, 8), (64, 16), (128, 2), (128, 8),
                  (128, 13), (128, 16), (256, 2), (256, 4), (256, 7),
                  (256, 8), (256, 16), (512, 2), (512, 4), (512, 8),
                  (512, 16), (1024, 1), (1024, 2), (1024, 4), (1024, 8)]
WIDE_EXTRA = {("plain", "f32"), ("tail", "f32")}
VEC = {"f32": 4, "bf16": 8, "f16": 8}   # elements per 128-bit vector


# ---------------------------------------------------------------------------
# Every configuration, full size, automatic shape (what the benchmark runs)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", [k for k, c in gen.CONFIGS.items()
                                  if c.kind in ("plain", "tail")])
def test_config_full_size(oracle, name):
    cfg = gen.CONFIGS[name]
    say(f"config {name} rows={cfg.rows} n={cfg.n} {cfg.dtype}")
    inp = gen.make(cfg)
    if cfg.kind == "plain":
        got, _ = run_plain(inp)
        check_plain(oracle, inp, got, name)
    else:
        h, y = run_tail(inp)
        check_tail(oracle, inp, h, y, name)


# ---------------------------------------------------------------------------
# Every compiled shape, forced, on a row that leaves part of its tile empty
# ---------------------------------------------------------------------------
def _shape_cases():
    cases = []
    for op, st in (("plain", "f32"), ("plain", "bf16"), ("tail", "f32")):
        shapes = list(ROWTILE_SHAPES)
        if (op, st) in WIDE_EXTRA:
            shapes.append((1024, 16))
        for g, vpt in shapes:
            for ragged in (False, True):
                cases.append((op, st, g, vpt, ragged))
    return cases


def _case_id(c):
    return "{}-{}-g{}-v{}-{}".format(*c[:4], "ragged" if c[4] else "whole")


@pytest.mark.parametrize("case", _shape_cases(), ids=_case_id)
def test_forced_rowtile_shape(oracle, case):
    """Every compiled shape on a row that leaves part of its tile empty; the
    ragged variant adds the largest remainder (W - 1 elements past the last
    whole vector)."""
    op, st, g, vpt, ragged = case
    w = VEC[st]
    nv = max(1, g * vpt - g // 2 - (1 if g == 1 else 0))
    n = nv * w + (w - 1 if ragged else 0)
    rows = 37
    seed = 1000 + g * 31 + vpt + (7 if ragged else 0)
    say(f"forced rowtile {_case_id(case)} rows={rows} n={n}")
    with snr.forced_shape("rowtile", g, vpt):
        if op == "plain":
            inp = gen.random_plain(rows, n, seed, dtype=st)
            got, _ = run_plain(inp)
            shape = snr.last_shape()
            check_plain(oracle, inp, got, _case_id(case))
        else:
            inp = gen.random_tail(rows, n, seed)
            h, y = run_tail(inp)
            shape = snr.last_shape()
            check_tail(oracle, inp, h, y, _case_id(case))
    assert shape == f"rowtile:{g}:{vpt}:{w}", shape


@pytest.mark.parametrize("op", ["plain", "tail"])
@pytest.mark.parametrize("ragged", [False, True])
@pytest.mark.parametrize("chunks_nv", [(1, 0), (1, 100), (3, 2 * 1024 + 5),
                                       (5, 5 * 1024)])
def test_forced_split(oracle, op, ragged, chunks_nv):
    chunks, nv = chunks_nv
    n = nv * 4 + (3 if ragged else 0)
    if n == 0:
        n = 1
    rows = 7
    say(f"forced split op={op} ragged={ragged} chunks={chunks} rows={rows} "
        f"n={n}")
    with snr.forced_shape("split", 0, 8):
        if op == "plain":
            inp = gen.random_plain(rows, n, 77 + chunks + n)
            got, _ = run_plain(inp)
            shape = snr.last_shape()
            check_plain(oracle, inp, got, f"split-{op}-n{n}")
        else:
            inp = gen.random_tail(rows, n, 78 + chunks + n)
            h, y = run_tail(inp)
            shape = snr.last_shape()
            check_tail(oracle, inp, h, y, f"split-{op}-n{n}")
    assert shape == f"split:256:4:4:{chunks}", shape
    assert snr.split_timeouts() == 0


@pytest.mark.parametrize("name", ["edge_256x65536_f32", "edge_256x16384_f32"])
def test_split_full_size(oracle, name):
    """The split-row reduction on the edge sweep's widest rows at full size
    (the automatic choice there is a 1024-lane register tile)."""
    cfg = gen.CONFIGS[name]
    say(f"split full size {name}")
    inp = gen.make(cfg)
    with snr.forced_shape("split", 0, 8):
        got, _ = run_plain(inp)
        shape = snr.last_shape()
    check_plain(oracle, inp, got, f"split-{name}")
    assert shape.startswith("split:256:4:4:")
    tin = gen.random_tail(64, cfg.n, 9100 + cfg.n)
    with snr.forced_shape("split", 0, 8):
        h, y = run_tail(tin)
    check_tail(oracle, tin, h, y, f"split-tail-{cfg.n}")
    assert snr.split_timeouts() == 0


@pytest.mark.parametrize("op_st", [("plain", "f32"), ("plain", "bf16"),
                                   ("tail", "f32")])
@pytest.mark.parametrize("n", [1, 3, 100, 6657, 2048 * 8 * 3 + 5])
def test_forced_multipass(oracle, op_st, n):
    op, st = op_st
    w = VEC[st]
    rows = 7
    chunks = max(1, -(-(n // w) // 4096))
    say(f"forced multipass {op} {st} rows={rows} n={n}")
    with snr.forced_shape("multipass"):
        if op == "plain":
            inp = gen.random_plain(rows, n, 9900 + n, dtype=st)
            got, _ = run_plain(inp)
            shape = snr.last_shape()
            check_plain(oracle, inp, got, f"multipass-{op}-{st}-{n}")
        else:
            inp = gen.random_tail(rows, n, 9901 + n)
            h, y = run_tail(inp)
            shape = snr.last_shape()
            check_tail(oracle, inp, h, y, f"multipass-tail-{n}")
    assert shape == f"multipass:256:16:{w}:{chunks}", shape


@pytest.mark.parametrize("op_st_n", [("plain", "f32", 8192 * 1024 + 5),
                                     ("tail", "f32", 8192 * 1024 + 5),
                                     ("plain", "bf16", 8 * 2048 * 1025 + 3)])
def test_rows_wider_than_the_split_capacity(oracle, op_st_n):
    """Rows too wide for co-resident chunks fall back to the multi-pass
    kernels automatically."""
    op, st, n = op_st_n
    rows = 2
    say(f"very wide {op} {st} rows={rows} n={n}")
    if op == "plain":
        inp = gen.random_plain(rows, n, 9950, dtype=st)
        got, _ = run_plain(inp)
        shape = snr.last_shape()
        check_plain(oracle, inp, got, f"wide-{op}-{st}")
    else:
        inp = gen.random_tail(rows, n, 9951)
        h, y = run_tail(inp)
        shape = snr.last_shape()
        check_tail(oracle, inp, h, y, "wide-tail")
    assert shape.startswith("multipass:256:16:"), shape


def test_forced_shape_that_cannot_hold_the_row_is_refused():
    x = torch.zeros(4, 4096, device=DEV)
    g = torch.ones(4096, device=DEV)
    with snr.forced_shape("rowtile", 64, 2):
        with pytest.raises(snr.SnrError) as ei:
            snr.rmsnorm_fwd(x, g, 1e-5)
    assert ei.value.code == _lib.SNR_ERR_SHAPE
    with snr.forced_shape("rowtile", 3, 4):
        with pytest.raises(snr.SnrError):
            snr.rmsnorm_fwd(x, g, 1e-5)


# ---------------------------------------------------------------------------
# Ragged and misaligned rows, automatic shape
# ---------------------------------------------------------------------------
RAGGED_N = [1, 2, 3, 4, 5, 7, 8, 63, 65, 127, 129, 255, 257, 1000, 1023,
            4097, 6657, 16385, 33333, 100003]


@pytest.mark.parametrize("n", RAGGED_N)
def test_ragged_plain(oracle, n):
    rows = 67
    say(f"ragged plain rows={rows} n={n}")
    inp = gen.random_plain(rows, n, 3000 + n, lo=-6, hi=4)
    got, _ = run_plain(inp)
    check_plain(oracle, inp, got, f"ragged-plain-{n}")
    inpb = gen.random_plain(rows, n, 4000 + n, dtype="bf16")
    gotb, _ = run_plain(inpb)
    check_plain(oracle, inpb, gotb, f"ragged-plain-bf16-{n}")


@pytest.mark.parametrize("n", RAGGED_N)
def test_ragged_tail(oracle, n):
    rows = 29
    say(f"ragged tail rows={rows} n={n}")
    inp = gen.random_tail(rows, n, 5000 + n)
    h, y = run_tail(inp)
    check_tail(oracle, inp, h, y, f"ragged-tail-{n}")


@pytest.mark.parametrize("n", [6656, 768, 4096])
def test_misaligned_base_pointer(oracle, n):
    """A view one element into its allocation is not 16-byte aligned: rows
    still move with 128-bit accesses and give the aligned result exactly."""
    rows = 16
    say(f"misaligned rows={rows} n={n}")
    inp = gen.random_plain(rows, n, 6000 + n)
    buf = torch.empty(rows * n + 1, device=DEV)
    x = buf[1:].view(rows, n)
    x.copy_(dev(inp["x"], "f32"))
    gbuf = torch.empty(n + 1, device=DEV)
    g = gbuf[1:]
    g.copy_(dev(inp["gamma"], "f32"))
    ybuf = torch.full((rows * n + 1,), float("nan"), device=DEV)
    y = ybuf[1:].view(rows, n)
    snr.rmsnorm_fwd(x, g, inp["eps"], out=y)
    torch.cuda.synchronize()
    misaligned = host_f64(y)
    assert snr.last_shape().endswith(":4"), snr.last_shape()
    check_plain(oracle, inp, misaligned, f"misaligned-{n}")
    # the same rows from an aligned allocation give the same bits
    got, _ = run_plain(inp)
    assert np.array_equal(got, misaligned)


# ---------------------------------------------------------------------------
# In place, sentinels, determinism, rows = 0, streams
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [6656, 6657, 65536, 3])
def test_in_place(oracle, n):
    rows = 9
    say(f"in-place rows={rows} n={n}")
    inp = gen.random_plain(rows, n, 7000 + n)
    got, _ = run_plain(inp, out_is_x=True)
    check_plain(oracle, inp, got, f"in-place-plain-{n}")
    tin = gen.random_tail(rows, n, 7100 + n)
    h, y = run_tail(tin, in_place=True)
    check_tail(oracle, tin, h, y, f"in-place-tail-{n}")


@pytest.mark.parametrize("prefill", [float("nan"), -999.0])
@pytest.mark.parametrize("n", [2, 3, 6657, 65536])
def test_sentinel_prefill_is_overwritten(oracle, prefill, n):
    rows = 5
    say(f"sentinel {prefill} rows={rows} n={n}")
    inp = gen.random_plain(rows, n, 8000 + n)
    got, _ = run_plain(inp, prefill=prefill)
    assert not np.any(got == prefill) or prefill != prefill
    assert np.all(np.isfinite(got))
    check_plain(oracle, inp, got, f"sentinel-{n}")
    tin = gen.random_tail(rows, n, 8100 + n)
    h, y = run_tail(tin, prefill=prefill)
    assert np.all(np.isfinite(h)) and np.all(np.isfinite(y))
    check_tail(oracle, tin, h, y, f"sentinel-tail-{n}")


@pytest.mark.parametrize("name", ["tail_4096x6656_f32", "edge_256x65536_f32",
                                  "plain_16384x4096_bf16", "edge_256x3_f32"])
def test_bitwise_deterministic(name):
    cfg = gen.CONFIGS[name]
    say(f"determinism {name}")
    inp = gen.make(cfg)
    if cfg.kind == "plain":
        a, _ = run_plain(inp)
        b, _ = run_plain(inp)
        assert np.array_equal(a, b)
    else:
        h1, y1 = run_tail(inp)
        h2, y2 = run_tail(inp)
        assert np.array_equal(h1, h2) and np.array_equal(y1, y2)


@pytest.mark.parametrize("op,rows,n", [("plain", 1024, 65536),
                                        ("tail", 512, 65536),
                                        ("plain", 2000, 3 * 1024 * 4 + 5)])
def test_split_repeated_runs_are_identical(oracle, op, rows, n):
    """The split-row kernel is the one path whose workgroups wait on one
    another. With more rows than can be co-resident (each workgroup walks
    several rows), 40 back-to-back runs must give bit-identical outputs that
    match the oracle, and no wait may have given up."""
    say(f"split repeated op={op} rows={rows} n={n}")
    if op == "plain":
        inp = gen.random_plain(rows, n, 9300 + rows)
        x, g = dev(inp["x"], "f32"), dev(inp["gamma"], "f32")
        outs = [torch.full_like(x, float("nan"))]
        call = lambda: snr.rmsnorm_fwd(x, g, inp["eps"], out=outs[0])  # noqa: E731
    else:
        inp = gen.random_tail(rows, n, 9400 + rows)
        a, r = dev(inp["a"], "f32"), dev(inp["r"], "f32")
        gp, gq = dev(inp["gamma_post"], "f32"), dev(inp["gamma_pre"], "f32")
        outs = [torch.full_like(a, float("nan")), torch.full_like(a, float("nan"))]
        call = lambda: snr.sandwich_tail(a, r, gp, inp["eps_post"], gq,  # noqa: E731
                                         inp["eps_pre"], h_out=outs[0],
                                         y_out=outs[1])
    with snr.forced_shape("split", 0, 8):
        call()
        shape = snr.last_shape()
        first = [o.clone() for o in outs]
        for _ in range(39):
            for o in outs:
                o.fill_(float("nan"))
            call()
            torch.cuda.synchronize()
            for o, f in zip(outs, first):
                assert torch.equal(o, f)
    assert shape.startswith("split:256:4:4:"), shape
    assert snr.split_timeouts() == 0
    if op == "plain":
        check_plain(oracle, inp, host_f64(first[0]), f"split-repeat-{n}")
    else:
        check_tail(oracle, inp, host_f64(first[0]), host_f64(first[1]),
                   f"split-repeat-tail-{n}")


@pytest.mark.parametrize("n", [6656, 6657, 3])
def test_subnormal_epsilon(oracle, n):
    """epsilon = the smallest f32 subnormal (2^-149) on both norms: zero rows
    give exactly 0 and h = r, and rows whose mean square plus epsilon is
    below the smallest normal match the oracle."""
    say(f"subnormal epsilon n={n}")
    eps = float(np.float32(2.0 ** -149))
    inp = gen.random_plain(6, n, 9500 + n)
    inp["eps"] = eps
    x = inp["x"]
    x[0] = 0.0
    x[1] = 0.0
    x[1, n // 2] = np.float32(1e-18)      # mean square below 2^-126
    got, _ = run_plain(inp)
    check_plain(oracle, inp, got, f"subnormal-eps-plain-{n}")
    assert not got[0].any()
    tin = gen.random_tail(4, n, 9600 + n)
    tin["eps_post"] = tin["eps_pre"] = eps
    tin["a"][0] = 0.0                     # h = r, y = rmsnorm(r)
    tin["a"][1] = 0.0
    tin["r"][1] = 0.0                     # h = 0, y = 0
    tin["a"][2] = 0.0
    tin["a"][2, 0] = np.float32(1e-18)
    tin["r"][2] = 0.0                     # h and y from a tiny post-norm
    h, y = run_tail(tin)
    check_tail(oracle, tin, h, y, f"subnormal-eps-tail-{n}")
    assert np.array_equal(h[0], tin["r"][0].astype(np.float64))
    assert not h[1].any() and not y[1].any()


@pytest.mark.parametrize("shape,n,op", [("split", 4096 * 1024, "plain"),
                                        ("split", 700 * 4096, "tail"),
                                        ("multipass", 16384 * 1024, "plain"),
                                        ("multipass", 4 * 8192 * 1024 + 5,
                                         "plain")])
def test_wide_constant_rows(oracle, shape, n, op):
    """Constant rows cut into 700 to 2049 chunks: every chunk's partial sum
    of squares is the same, which is where adding the partials in one chain
    drifts by about a rounding per addition (1e-5 of the sum at 1024
    chunks). Added in blocks of 32 they stay within 2e-6 of the exact
    result."""
    say(f"wide constant rows {shape} {op} n={n}")
    rows = 2
    if op == "plain":
        x = np.empty((rows, n), np.float32)
        x[0], x[1] = np.float32(0.7), np.float32(-1.1)
        g = np.full(n, np.float32(1.3))
        inp = {"x": x, "gamma": g, "eps": 1e-5, "dtype": "f32"}
        with snr.forced_shape(shape, 0, 8):
            got, _ = run_plain(inp)
            sh = snr.last_shape()
        want = oracle.rmsnorm(x, g, 1e-5)
        from parity import plain_error
        err = plain_error(got, want)
    else:
        a = np.empty((rows, n), np.float32)
        r = np.empty((rows, n), np.float32)
        a[0], a[1] = np.float32(0.3), np.float32(2.5)
        r[0], r[1] = np.float32(-0.9), np.float32(0.1)
        gp, gq = np.full(n, np.float32(1.1)), np.full(n, np.float32(0.7))
        inp = {"a": a, "r": r, "gamma_post": gp, "gamma_pre": gq,
               "eps_post": 1e-8, "eps_pre": 1e-5, "dtype": "f32"}
        with snr.forced_shape(shape, 0, 8):
            h, y = run_tail(inp)
            sh = snr.last_shape()
        from parity import tail_errors
        o = oracle.sandwich_tail(a, r, gp, 1e-8, gq, 1e-5)
        err = max(tail_errors(h, y, o, r, gq))
    say(f"  {sh}: max rel err {err:.3e}")
    assert sh.startswith(shape + ":"), sh
    assert err < 2e-6, err
    assert snr.split_timeouts() == 0


def test_rows_zero_is_a_noop():
    say("rows=0")
    x = torch.empty(0, 64, device=DEV)
    g = torch.ones(64, device=DEV)
    y = snr.rmsnorm_fwd(x, g, 1e-5)
    assert y.shape == (0, 64)
    h, yy = snr.sandwich_tail(x, x, g, 1e-8, g, 1e-5)
    assert h.shape == (0, 64) and yy.shape == (0, 64)


def test_non_default_stream(oracle):
    say("non-default stream")
    inp = gen.make("tail_8x6656_f32")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a, r = dev(inp["a"], "f32"), dev(inp["r"], "f32")
        gp, gq = dev(inp["gamma_post"], "f32"), dev(inp["gamma_pre"], "f32")
        h, y = snr.sandwich_tail(a, r, gp, inp["eps_post"], gq,
                                 inp["eps_pre"])
    s.synchronize()
    check_tail(oracle, inp, host_f64(h), host_f64(y), "stream")


def test_bf16_output_is_round_to_nearest_even(oracle):
    """8e-3 cannot tell rounding from truncation (both stay within one bf16
    unit), so check the rounding itself: almost every output equals the
    oracle's value rounded to nearest-even, and none is more than one bf16
    unit away."""
    say("bf16 rounding")
    inp = gen.make("plain_16384x4096_bf16", rows=512)
    x, g = dev(inp["x"], "bf16"), dev(inp["gamma"], "bf16")
    y = snr.rmsnorm_fwd(x, g, inp["eps"])
    torch.cuda.synchronize()
    bits = y.view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle.rmsnorm(inp["x"], inp["gamma"], inp["eps"])
    want_bits = gen.f32_to_bf16_bits(want.astype(np.float32))
    ulps = np.abs(bits.astype(np.int32) - want_bits.astype(np.int32))
    # same sign everywhere (the sign bit would make the difference huge)
    assert ulps.max() <= 1, ulps.max()
    assert np.mean(ulps == 0) >= 0.999, np.mean(ulps == 0)


def test_split_wait_budget_exhausted_is_reported_and_recovered(oracle,
                                                              monkeypatch):
    """Force the split-row kernel's bounded wait to give up (a budget of no
    polls): the kernel still finishes, its outputs are NaN, the overrun is
    counted, and the next call with the normal budget is correct again."""
    rows, n = 64, 5 * 2048 * 4
    say(f"split watchdog rows={rows} n={n}")
    inp = gen.random_plain(rows, n, 4242)
    assert snr.split_timeouts() == 0
    monkeypatch.setenv("SNR_SPLIT_SPIN_LIMIT", "0")
    with snr.forced_shape("split", 0, 8):
        bad, _ = run_plain(inp)
        assert np.isnan(bad).all()
        assert snr.split_timeouts() > 0
        monkeypatch.delenv("SNR_SPLIT_SPIN_LIMIT")
        got, _ = run_plain(inp)
    assert snr.split_timeouts() == 0
    check_plain(oracle, inp, got, "split-after-watchdog")
