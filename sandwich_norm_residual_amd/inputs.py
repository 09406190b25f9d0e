"""Seeded synthetic inputs for RMSNorm and the dual-epsilon sandwich tail.

This module is shared by the GPU path's tests and benchmark and by the oracle's
tests. It draws random numbers, lays out arrays, and scales each edge-sweep
row to its drawn target mean square (the input recipe); it contains none of
the method's arithmetic (no epsilon, no normalised output, no gain applied).

The workloads stand in for the residual stream of the model the Muser book
describes (hidden width n = 6656, section 12.1 of "RMSNorm and the
dual-epsilon sandwich"): real activations need that model's weights, which are
not available, so each configuration draws Gaussian rows with a log-uniform
per-row scale, and per-channel gains gamma = 1 + 0.1 * N(0, 1).

Every array comes from ``numpy.random.Generator(PCG64(seed))``; the order of
draws within a configuration is fixed, so a seed names the data exactly.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = np.float32


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# -- bf16 storage helpers (encode for input preparation, exact decode) -------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and return
    the 16-bit patterns as uint16. NaN stays NaN (quietened)."""
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(nan, ((u >> 16) | 0x40) & 0xFFFF, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(F32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (nearest even) as uint16 bits."""
    return np.ascontiguousarray(x, dtype=F32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of binary16 bit patterns to float32."""
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(F32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values in a storage type: float32 itself, or the 16-bit
    patterns (uint16) of bf16 / f16."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=F32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    raise ValueError(dtype)


def from_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 values of a storage array."""
    if dtype == "f32":
        return np.asarray(x, dtype=F32)
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    if dtype == "f16":
        return f16_bits_to_f32(x)
    raise ValueError(dtype)


# -- configurations ------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    name: str
    kind: str            # "plain", "tail", "norm_add", "add_norm", "multi"
    rows: int
    n: int
    dtype: str           # "f32", "bf16" or "f16" (storage type)
    seed: int
    eps: tuple           # (eps,) for plain; (eps_post, eps_pre) for tail
    scale_exp: tuple = ()   # per-row log10 scale range(s)
    edge: bool = False   # structured rows 0-5 + log-uniform mean-square
    segments: tuple = ()  # rows of each problem of a several-norm workload
    notes: str = field(default="", compare=False)


EPS_PRE = 1e-5    # pre-norm epsilon (the checkpoint's value)
EPS_POST = 1e-8   # post-norm epsilon (hard-coded in the sandwich's post norms)

EDGE_NS = (2, 3, 768, 2048, 6657, 16384, 65536)


def _configs() -> dict:
    c = {}

    def add(cfg: Config):
        c[cfg.name] = cfg

    add(Config("plain_64x6656_f32", "plain", 64, 6656, "f32", 101, (1e-5,),
               ((-2.0, 1.0),)))
    add(Config("tail_1x6656_f32", "tail", 1, 6656, "f32", 201,
               (EPS_POST, EPS_PRE), ((-3.0, 2.0), (-1.0, 1.0))))
    add(Config("tail_8x6656_f32", "tail", 8, 6656, "f32", 208,
               (EPS_POST, EPS_PRE), ((-3.0, 2.0), (-1.0, 1.0))))
    add(Config("tail_4096x6656_f32", "tail", 4096, 6656, "f32", 301,
               (EPS_POST, EPS_PRE), ((-3.0, 2.0), (-1.0, 1.0))))
    add(Config("plain_16384x4096_bf16", "plain", 16384, 4096, "bf16", 401,
               (1e-6,), ((-2.0, 2.0),)))
    # the tail in 16-bit storage, and its two halves on their own
    add(Config("tail_4096x6656_bf16", "tail", 4096, 6656, "bf16", 302,
               (EPS_POST, EPS_PRE), ((-3.0, 2.0), (-1.0, 1.0))))
    add(Config("tail_4096x6656_f16", "tail", 4096, 6656, "f16", 303,
               (EPS_POST, EPS_PRE), ((-3.0, 2.0), (-1.0, 1.0))))
    add(Config("norm_add_4096x6656_f32", "norm_add", 4096, 6656, "f32", 311,
               (EPS_POST,), ((-3.0, 2.0), (-1.0, 1.0))))
    add(Config("add_norm_4096x6656_f32", "add_norm", 4096, 6656, "f32", 321,
               (EPS_PRE,), ((-1.0, 1.0), (-3.0, 2.0))))
    # per-head query and key norms of one layer (head_dim 128; 52 query and
    # 8 key heads per token): one token, and a 512-token prefill
    add(Config("qknorm_decode_f32", "multi", 60, 128, "f32", 331, (1e-5,),
               ((-2.0, 1.0),), segments=(52, 8)))
    add(Config("qknorm_prefill_bf16", "multi", 512 * 60, 128, "bf16", 332,
               (1e-5,), ((-2.0, 2.0),), segments=(512 * 52, 512 * 8)))
    # RMSNorm into Q8_1 records (n a multiple of 32): a 4096-token batch at
    # the model width, in f32 and bf16; one decode token at width 2560; and
    # an edge sweep (zero rows and blocks, spikes, tiny rows)
    add(Config("q8_4096x6656_f32", "q8", 4096, 6656, "f32", 341, (1e-5,),
               ((-2.0, 1.0),)))
    add(Config("q8_4096x6656_bf16", "q8", 4096, 6656, "bf16", 342, (1e-5,),
               ((-2.0, 1.0),)))
    add(Config("q8_1x2560_f32", "q8", 1, 2560, "f32", 343, (1e-5,),
               ((-2.0, 1.0),)))
    add(Config("q8_edge_256x6656_f32", "q8", 256, 6656, "f32", 344, (1e-5,),
               ((-12.0, 6.0),), edge=True))
    for n in EDGE_NS:
        add(Config(f"edge_256x{n}_f32", "plain", 256, n, "f32", 500 + n,
                   (1e-5,), ((-12.0, 6.0),), edge=True))
    # rows wider than any register tile (65536 elements): the split-row
    # kernels, with the plain norm's and the tail's recipes
    add(Config("plain_256x262144_f32", "plain", 256, 262144, "f32", 351,
               (1e-5,), ((-2.0, 1.0),)))
    add(Config("tail_256x262144_f32", "tail", 256, 262144, "f32", 352,
               (EPS_POST, EPS_PRE), ((-3.0, 2.0), (-1.0, 1.0))))
    add(Config("plain_16x1048576_f32", "plain", 16, 1048576, "f32", 353,
               (1e-5,), ((-2.0, 1.0),)))
    add(Config("tail_16x1048576_f32", "tail", 16, 1048576, "f32", 354,
               (EPS_POST, EPS_PRE), ((-3.0, 2.0), (-1.0, 1.0))))
    return c


CONFIGS = _configs()
HEADLINE = "tail_4096x6656_f32"


def _gamma(rng: np.random.Generator, n: int) -> np.ndarray:
    return (1.0 + 0.1 * rng.standard_normal(n)).astype(F32)


def _scaled_normal(rng, rows, n, lo, hi) -> np.ndarray:
    """Rows of N(0,1) times a per-row scale 10**U(lo, hi)."""
    scale = 10.0 ** rng.uniform(lo, hi, rows)
    z = rng.standard_normal((rows, n))
    z *= scale[:, None]
    return z.astype(F32)


def _edge_rows(rng, rows, n, lo, hi):
    """Edge-sweep rows and their target mean squares: row i has target
    mean-square m_i = 10**U(lo, hi) and is z * sqrt(m_i / mean(z^2)) with z
    drawn N(0,1), so its mean square is m_i up to the final rounding to f32.
    Rows 0-5 are structured (their targets are not used): all zero, constant
    +c, constant -c, alternating +-c, a one-hot spike, and a row at the
    smallest target mean-square 10**lo."""
    m = 10.0 ** rng.uniform(lo, hi, rows)
    z = rng.standard_normal((rows, n))
    ms = np.mean(z * z, axis=1)
    z *= np.sqrt(m / ms)[:, None]
    x = z.astype(F32)
    c = 1.5
    if rows > 0:
        x[0] = 0.0
    if rows > 1:
        x[1] = c
    if rows > 2:
        x[2] = -c
    if rows > 3:
        x[3] = np.where(np.arange(n) % 2 == 0, c, -c)
    if rows > 4:
        x[4] = 0.0
        x[4, n // 2] = 100.0
    if rows > 5:
        z5 = rng.standard_normal(n)
        x[5] = (z5 * np.sqrt(10.0 ** lo / np.mean(z5 * z5))).astype(F32)
    return x, m


def make_plain(cfg: Config, rows: int | None = None) -> dict:
    """Inputs for a plain RMSNorm configuration. ``rows`` may shrink the row
    count (the first rows of the same stream are NOT guaranteed identical to
    the full draw; a smaller row count is its own seeded input)."""
    assert cfg.kind in ("plain", "q8")
    rows = cfg.rows if rows is None else rows
    rng = rng_for(cfg.seed)
    gamma = _gamma(rng, cfg.n)
    lo, hi = cfg.scale_exp[0]
    out = {}
    if cfg.edge:
        x, out["target_ms"] = _edge_rows(rng, rows, cfg.n, lo, hi)
    else:
        x = _scaled_normal(rng, rows, cfg.n, lo, hi)
    out.update({"x": to_storage(x, cfg.dtype),
                "gamma": to_storage(gamma, cfg.dtype), "eps": cfg.eps[0],
                "dtype": cfg.dtype})
    return out


def make_tail(cfg: Config, rows: int | None = None) -> dict:
    """Inputs for a sandwich-tail configuration: block output a, residual r,
    the two gains and the two epsilons."""
    assert cfg.kind == "tail"
    rows = cfg.rows if rows is None else rows
    rng = rng_for(cfg.seed)
    gamma_post = _gamma(rng, cfg.n)
    gamma_pre = _gamma(rng, cfg.n)
    (alo, ahi), (rlo, rhi) = cfg.scale_exp
    a = _scaled_normal(rng, rows, cfg.n, alo, ahi)
    r = _scaled_normal(rng, rows, cfg.n, rlo, rhi)
    st = cfg.dtype
    return {"a": to_storage(a, st), "r": to_storage(r, st),
            "gamma_post": to_storage(gamma_post, st),
            "gamma_pre": to_storage(gamma_pre, st),
            "eps_post": cfg.eps[0], "eps_pre": cfg.eps[1], "dtype": st}


def make_pair(cfg: Config, rows: int | None = None) -> dict:
    """Inputs for norm_add (a = block output, b = residual) and add_norm
    (a = residual, b = block output): two rows streams, one gain, one eps."""
    assert cfg.kind in ("norm_add", "add_norm")
    rows = cfg.rows if rows is None else rows
    rng = rng_for(cfg.seed)
    gamma = _gamma(rng, cfg.n)
    (alo, ahi), (blo, bhi) = cfg.scale_exp
    a = _scaled_normal(rng, rows, cfg.n, alo, ahi)
    b = _scaled_normal(rng, rows, cfg.n, blo, bhi)
    st = cfg.dtype
    return {"a": to_storage(a, st), "b": to_storage(b, st),
            "gamma": to_storage(gamma, st), "eps": cfg.eps[0], "dtype": st}


def make_multi(cfg: Config) -> dict:
    """Inputs for a several-norm workload: one (x, gamma) per segment, all of
    width n, drawn in segment order."""
    assert cfg.kind == "multi"
    rng = rng_for(cfg.seed)
    lo, hi = cfg.scale_exp[0]
    xs, gs = [], []
    for rows in cfg.segments:
        gs.append(to_storage(_gamma(rng, cfg.n), cfg.dtype))
        xs.append(to_storage(_scaled_normal(rng, rows, cfg.n, lo, hi),
                             cfg.dtype))
    return {"xs": xs, "gammas": gs, "eps": cfg.eps[0], "dtype": cfg.dtype}


def make(cfg_or_name, rows: int | None = None) -> dict:
    cfg = CONFIGS[cfg_or_name] if isinstance(cfg_or_name, str) else cfg_or_name
    if cfg.kind in ("plain", "q8"):
        return make_plain(cfg, rows)
    if cfg.kind == "tail":
        return make_tail(cfg, rows)
    if cfg.kind == "multi":
        return make_multi(cfg)
    return make_pair(cfg, rows)


def random_pair(kind: str, rows: int, n: int, seed: int,
                dtype: str = "f32") -> dict:
    """Ad-hoc inputs for norm_add / add_norm sweeps."""
    cfg = Config(f"adhoc_{kind}_{rows}x{n}", kind, rows, n, dtype, seed,
                 (EPS_POST if kind == "norm_add" else EPS_PRE,),
                 ((-3.0, 2.0), (-1.0, 1.0)))
    return make_pair(cfg)


def random_plain(rows: int, n: int, seed: int, lo: float = -3.0,
                 hi: float = 3.0, dtype: str = "f32") -> dict:
    """Ad-hoc plain inputs for shape sweeps (same recipe as the configs)."""
    cfg = Config(f"adhoc_{rows}x{n}", "plain", rows, n, dtype, seed, (1e-5,),
                 ((lo, hi),))
    return make_plain(cfg)


def random_tail(rows: int, n: int, seed: int, dtype: str = "f32") -> dict:
    """Ad-hoc tail inputs for shape sweeps (same recipe as the configs)."""
    cfg = Config(f"adhoc_tail_{rows}x{n}", "tail", rows, n, dtype, seed,
                 (EPS_POST, EPS_PRE), ((-3.0, 2.0), (-1.0, 1.0)))
    return make_tail(cfg)
