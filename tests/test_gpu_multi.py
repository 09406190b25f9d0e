"""GPU parity of rmsnorm_fwd_multi: several RMSNorms of one row width in one
launch (the per-head query and key norms of a layer are the use the Muser
book's per-token dispatch count singles out), each segment against the f64
oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import check_plain, dev, host_f64, say  # noqa: E402

pytestmark = pytest.mark.gpu
AUTO_ROWTILE = [(1, 4), (2, 4), (4, 4), (8, 4), (16, 4), (32, 4), (128, 2),
                (128, 8), (256, 2), (256, 4), (512, 2), (512, 4), (1024, 1),
                (1024, 2), (1024, 4), (1024, 8)]


def run_multi(oracle, specs, st, label, in_place=()):
    """specs: list of (rows, n, eps, seed). Runs one multi call and checks
    every segment."""
    inps = []
    probs, outs = [], []
    for i, (rows, n, eps, seed) in enumerate(specs):
        inp = gen.random_plain(rows, n, seed, dtype=st)
        inp["eps"] = eps
        inps.append(inp)
        x = dev(inp["x"], st)
        g = dev(inp["gamma"], st)
        probs.append((x, g, eps))
        outs.append(x if i in in_place else torch.full_like(x, float("nan")))
    res = snr.rmsnorm_fwd_multi(probs, outs)
    torch.cuda.synchronize()
    shape = snr.last_shape()
    for i, (inp, y) in enumerate(zip(inps, res)):
        check_plain(oracle, inp, host_f64(y), f"{label}-seg{i}")
    return shape


@pytest.mark.parametrize("st", ["f32", "bf16", "f16"])
def test_qk_norm_decode(oracle, st):
    """One token: 52 query heads and 8 key heads of width 128, own gains
    and epsilons, one launch."""
    say(f"qk decode {st}")
    shape = run_multi(oracle, [(52, 128, 1e-5, 31), (8, 128, 1e-6, 32)], st,
                      f"qk-decode-{st}")
    assert shape.startswith("multi:") and shape.endswith(":2"), shape


@pytest.mark.parametrize("st", ["f32", "bf16"])
def test_qk_norm_prefill(oracle, st):
    say(f"qk prefill {st}")
    shape = run_multi(oracle, [(512 * 52, 128, 1e-5, 41),
                               (512 * 8, 128, 1e-5, 42)], st,
                      f"qk-prefill-{st}")
    assert shape.startswith("multi:")


def test_eight_ragged_segments_with_in_place(oracle):
    specs = [(r, 6657, e, 50 + i) for i, (r, e) in enumerate(
        [(1, 1e-5), (7, 1e-8), (64, 1e-6), (3, 1e-5), (0, 1e-5), (130, 1e-5),
         (2, 1e-3), (33, 1e-5)])]
    say("eight segments")
    shape = run_multi(oracle, specs, "f32", "eight", in_place=(2, 5))
    assert shape.endswith(":8"), shape


def test_wide_rows_fall_back_to_one_launch_per_segment(oracle):
    say("multi wide rows")
    shape = run_multi(oracle, [(3, 100003, 1e-5, 61), (2, 100003, 1e-5, 62)],
                      "f32", "wide")
    assert not shape.startswith("multi:"), shape


@pytest.mark.parametrize("gv", AUTO_ROWTILE + [(1024, 16)])
def test_forced_shapes(oracle, gv):
    g, v = gv
    n = (max(1, g * v - g // 2 - (1 if g == 1 else 0))) * 4 + 3
    say(f"multi forced g={g} v={v} n={n}")
    with snr.forced_shape("rowtile", g, v):
        shape = run_multi(oracle, [(9, n, 1e-5, 70), (5, n, 1e-8, 71),
                                   (12, n, 1e-6, 72)], "f32",
                          f"multi-g{g}-v{v}")
    assert shape == f"multi:{g}:{v}:4:3", shape


def test_matches_separate_launches_bitwise():
    """Same shape, same rows: a segment of a multi launch gives the same bits
    as rmsnorm_fwd on that segment alone."""
    say("multi vs single")
    q = torch.randn(52, 128, device="cuda:0")
    k = torch.randn(8, 128, device="cuda:0")
    gq = torch.rand(128, device="cuda:0") + 0.5
    gk = torch.rand(128, device="cuda:0") + 0.5
    yq, yk = snr.rmsnorm_fwd_multi([(q, gq, 1e-5), (k, gk, 1e-5)])
    assert torch.equal(yq, snr.rmsnorm_fwd(q, gq, 1e-5))
    assert torch.equal(yk, snr.rmsnorm_fwd(k, gk, 1e-5))
