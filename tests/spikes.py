"""Rows that make the rounding of a stored intermediate show.

The tail's h = r + post-norm(a) and add_then_norm's s = a + b are stored in
the storage type and normalised again. In these rows one element of the
intermediate is a power of two 2^E plus just under half a unit of the storage
type (the spacing above 2^E), so storing it rounds it down by nearly a full
unit roundoff, and it dominates the row's mean of squares. The other
elements are ordinary and round by varying amounts. Normalising the rounded
copy therefore moves every output by the dominant element's rounding as well
as its own: up to three roundings in y. Test infrastructure; the values are
chosen in closed form and checked against the oracle by the CPU test.
"""
import numpy as np

from sandwich_norm_residual_amd import inputs as gen

SIGNIFICAND_BITS = {"bf16": 8, "f16": 11}
SPIKE_EXP = {"bf16": 18, "f16": 14}   # 2^E within the storage type's range


def unit_above(dtype):
    """The spacing of the storage type just above 2^E."""
    return 2.0 ** (SPIKE_EXP[dtype] - SIGNIFICAND_BITS[dtype] + 1)


def add_norm_spikes(rows, n, seed, dtype):
    """add_then_norm inputs: a[:, 0] = 2^E, b[:, 0] = 0.498 units."""
    rng = gen.rng_for(seed)
    a = rng.standard_normal((rows, n))
    b = 0.16 * rng.standard_normal((rows, n))
    a[:, 0] = 2.0 ** SPIKE_EXP[dtype]
    b[:, 0] = 0.498 * unit_above(dtype)
    g = 1.0 + 0.1 * rng.standard_normal(n)
    st = dtype
    return {"a": gen.to_storage(a.astype(np.float32), st),
            "b": gen.to_storage(b.astype(np.float32), st),
            "gamma": gen.to_storage(g.astype(np.float32), st),
            "eps": 1e-5, "dtype": st}


def tail_spikes(rows, n, seed, dtype):
    """Tail inputs: r[:, 0] = 2^E, and a one-hot-dominated a (a[:, 0] = 1,
    the rest 0.01 N(0,1)) whose post-norm at element 0 is about
    gamma_post[0] * sqrt(n) / sqrt(1 + 1e-4 (n - 1)); gamma_post[0] is set so
    that this is about 0.45 units, and the other elements of h are
    r_j + about 0.16 N(0,1)."""
    rng = gen.rng_for(seed)
    a = 0.01 * rng.standard_normal((rows, n))
    r = rng.standard_normal((rows, n))
    a[:, 0] = 1.0
    r[:, 0] = 2.0 ** SPIKE_EXP[dtype]
    gp = 1.0 + 0.1 * rng.standard_normal(n)
    gq = 1.0 + 0.1 * rng.standard_normal(n)
    gp[0] = 0.45 * unit_above(dtype) * np.sqrt(1.0 + 1e-4 * (n - 1)) / np.sqrt(n)
    st = dtype
    return {"a": gen.to_storage(a.astype(np.float32), st),
            "r": gen.to_storage(r.astype(np.float32), st),
            "gamma_post": gen.to_storage(gp.astype(np.float32), st),
            "gamma_pre": gen.to_storage(gq.astype(np.float32), st),
            "eps_post": 1e-8, "eps_pre": 1e-5, "dtype": st}
