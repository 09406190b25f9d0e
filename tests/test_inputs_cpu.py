"""The seeded input generator (sandwich_norm_residual_amd/inputs.py), on the
CPU: a seed names its data exactly, every configuration draws the
distributions it states (per-row scales, gains, the edge sweep's structured
rows and mean-square range), and the 16-bit storage helpers round to nearest
even and decode exactly (checked against torch's own conversions)."""
import numpy as np
import pytest

from sandwich_norm_residual_amd import inputs as gen

SMALL = ["plain_64x6656_f32", "tail_8x6656_f32", "edge_256x2_f32",
         "edge_256x6657_f32", "qknorm_decode_f32", "q8_1x2560_f32",
         "norm_add_4096x6656_f32"]


def _arrays(d):
    out = []
    for k in sorted(d):
        v = d[k]
        if isinstance(v, np.ndarray):
            out.append((k, v))
        elif isinstance(v, list):
            out.extend((f"{k}{i}", a) for i, a in enumerate(v))
    return out


@pytest.mark.parametrize("name", SMALL)
def test_a_seed_names_the_data(name):
    rows = 16 if gen.CONFIGS[name].rows > 256 else None
    a = _arrays(gen.make(name, rows) if rows else gen.make(name))
    b = _arrays(gen.make(name, rows) if rows else gen.make(name))
    assert [k for k, _ in a] == [k for k, _ in b]
    for (k, x), (_, y) in zip(a, b):
        assert x.dtype == y.dtype and np.array_equal(x, y), k


def test_different_seeds_differ():
    x = gen.random_plain(4, 256, 1)["x"]
    y = gen.random_plain(4, 256, 2)["x"]
    assert not np.array_equal(x, y)


def test_configs_are_distinct_and_well_formed():
    seeds = [c.seed for c in gen.CONFIGS.values()]
    assert len(seeds) == len(set(seeds))
    for c in gen.CONFIGS.values():
        assert c.rows >= 1 and c.n >= 1 and c.dtype in ("f32", "bf16", "f16")
        assert all(e > 0 for e in c.eps)
        if c.kind == "q8":
            assert c.n % 32 == 0
        if c.kind == "multi":
            assert sum(c.segments) == c.rows
    assert gen.HEADLINE in gen.CONFIGS


def _row_rms(x):
    x = x.astype(np.float64)
    return np.sqrt(np.mean(x * x, axis=1))


def _check_gain(g):
    g = g.astype(np.float64)
    assert abs(g.mean() - 1.0) < 0.01
    assert 0.09 < g.std() < 0.11


@pytest.mark.parametrize("name,key,lo,hi", [
    ("plain_64x6656_f32", "x", -2.0, 1.0),
    ("tail_8x6656_f32", "a", -3.0, 2.0),
    ("tail_8x6656_f32", "r", -1.0, 1.0),
])
def test_per_row_scales_are_in_the_stated_range(name, key, lo, hi):
    d = gen.make(name)
    rms = _row_rms(gen.from_storage(d[key], d["dtype"]))
    # N(0,1) * s over 6656 values: the row's rms is s within a few percent
    assert np.all(rms >= 10.0 ** lo * 0.95) and np.all(rms <= 10.0 ** hi * 1.05)
    for g in ("gamma", "gamma_post", "gamma_pre"):
        if g in d:
            _check_gain(gen.from_storage(d[g], d["dtype"]))


def test_headline_scales_span_the_range():
    """The 4096 rows of the headline draw a per-row scale log-uniform over
    10^[-3, 2] (a) and 10^[-1, 1] (r): both ends are reached."""
    d = gen.make("tail_4096x6656_f32", rows=512)
    la = np.log10(_row_rms(d["a"]))
    lr = np.log10(_row_rms(d["r"]))
    assert la.min() < -2.8 and la.max() > 1.8
    assert lr.min() < -0.9 and lr.max() > 0.9
    # log-uniform: each fifth of the range holds about a fifth of the rows
    counts, _ = np.histogram(la, bins=5, range=(-3, 2))
    assert counts.min() > 0.12 * len(la)


def test_bf16_config_values_are_bf16():
    d = gen.make("plain_16384x4096_bf16", rows=64)
    assert d["x"].dtype == np.uint16 and d["gamma"].dtype == np.uint16
    x = gen.from_storage(d["x"], "bf16")
    # every decoded value is exactly representable in bf16: low 16 bits zero
    assert not np.any(x.view(np.uint32) & 0xFFFF)
    rms = _row_rms(x)
    assert np.all(rms >= 1e-2 * 0.95) and np.all(rms <= 1e2 * 1.05)
    _check_gain(gen.from_storage(d["gamma"], "bf16"))


@pytest.mark.parametrize("n", [768, 6657, 16384])
def test_edge_rows(n):
    d = gen.make(f"edge_256x{n}_f32")
    x = d["x"].astype(np.float64)
    c = 1.5
    assert np.all(x[0] == 0.0)
    assert np.all(x[1] == c) and np.all(x[2] == -c)
    assert np.all(x[3, 0::2] == c) and np.all(x[3, 1::2] == -c)
    spike = np.zeros(n)
    spike[n // 2] = 100.0
    assert np.array_equal(x[4], spike)
    ms = np.mean(x * x, axis=1)
    # the tiny row sits at the smallest target mean square, up to rounding
    assert abs(ms[5] / 1e-12 - 1.0) < 1e-6
    rest = ms[6:]
    # every other row's realised mean square is its drawn target m (up to
    # the rounding of its elements to f32), log-uniform over 1e-12 .. 1e6
    m = d["target_ms"][6:]
    assert np.all(np.abs(rest / m - 1.0) < 1e-6)
    assert np.all(m >= 1e-12) and np.all(m <= 1e6)
    assert m.min() < 1e-9 and m.max() > 1e3


def test_small_edge_rows_keep_their_structure():
    for n in (2, 3):
        d = gen.make(f"edge_256x{n}_f32")
        x = d["x"]
        assert np.all(x[0] == 0) and np.all(x[1] == 1.5) and np.all(x[2] == -1.5)
        assert x[4, n // 2] == 100.0 and np.count_nonzero(x[4]) == 1
        # even two or three elements carry the drawn mean square exactly
        xd = x.astype(np.float64)
        ms = np.mean(xd[6:] * xd[6:], axis=1)
        assert np.all(np.abs(ms / d["target_ms"][6:] - 1.0) < 1e-6)


def test_bf16_rounds_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)      # bf16 spacing at 1.0
    half = np.float32(2.0 ** -8)
    vals = np.array([one + half,                 # tie, rounds down to even 1.0
                     one + ulp + half,           # tie, rounds up to 1 + 2 ulp
                     one + half + 2.0 ** -20,    # above the tie, rounds up
                     -(one + half),
                     np.inf, -np.inf, 0.0, -0.0], dtype=np.float32)
    got = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(vals))
    want = np.array([1.0, 1.0 + 2 * ulp, 1.0 + ulp, -1.0, np.inf, -np.inf,
                     0.0, -0.0], dtype=np.float32)
    assert np.array_equal(got, want)
    assert np.signbit(got[-1])
    nan = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(np.array([np.nan],
                                                              np.float32)))
    assert np.isnan(nan[0])


def test_16_bit_helpers_match_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(7))
    x = (rng.standard_normal(100000) *
         10.0 ** rng.uniform(-6, 6, 100000)).astype(np.float32)
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(gen.f32_to_bf16_bits(x), tb.view(np.uint16))
    th = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy()
    with np.errstate(over="ignore"):     # values past f16's range become inf
        h16 = gen.f32_to_f16_bits(x)
    assert np.array_equal(h16, th.view(np.uint16))
    bits = rng.integers(0, 1 << 16, 100000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # finite bf16 patterns
    dec = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    assert np.array_equal(gen.bf16_bits_to_f32(bits), dec.numpy())
