"""Shared helpers of the GPU parity tests: device copies of seeded inputs in
their storage type, decoding of outputs, and the oracle comparisons."""
import numpy as np
import torch

import sandwich_norm_residual_amd as snr
from sandwich_norm_residual_amd import inputs as gen
from parity import NORMAL_MIN, TOLS, plain_error, scaled_error, tail_errors

DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16,
            "f16": torch.float16}


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def dev(arr, dtype):
    """A storage array (float32, or uint16 bits of bf16/f16) on the GPU."""
    arr = np.ascontiguousarray(arr)
    if dtype == "f32":
        return torch.from_numpy(arr.astype(np.float32, copy=False)).to(DEV)
    t = torch.from_numpy(arr.view(np.int16)).to(DEV)
    return t.view(TORCH_DT[dtype])


def host_f64(t):
    """A GPU tensor's exact values as float64."""
    if t.dtype == torch.float32:
        return t.cpu().numpy().astype(np.float64)
    bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
    st = "bf16" if t.dtype == torch.bfloat16 else "f16"
    return gen.from_storage(bits, st).astype(np.float64)


def f32(inp, key):
    """Exact float32 values of an input array (what the oracle receives)."""
    return gen.from_storage(inp[key], inp["dtype"])


def check_plain(oracle, inp, got, label):
    want = oracle.rmsnorm(f32(inp, "x"), f32(inp, "gamma"), inp["eps"])
    tol = TOLS[inp["dtype"]]
    err = plain_error(got, want, NORMAL_MIN[inp["dtype"]])
    say(f"{label}: max rel err {err:.3e} (tol {tol:g}) shape "
        f"{snr.last_shape()}")
    assert err <= tol, (label, err)
    return err


def check_tail(oracle, inp, h, y, label):
    r = f32(inp, "r")
    gq = f32(inp, "gamma_pre")
    o = oracle.sandwich_tail(f32(inp, "a"), r, f32(inp, "gamma_post"),
                             inp["eps_post"], gq, inp["eps_pre"])
    eh, ey = tail_errors(h, y, o, r, gq, NORMAL_MIN[inp["dtype"]])
    tol = TOLS[inp["dtype"]]
    say(f"{label}: h err {eh:.3e} y err {ey:.3e} (tol {tol:g}) shape "
        f"{snr.last_shape()}")
    assert eh <= tol and ey <= tol, (label, eh, ey)


def check_norm_add(oracle, inp, out, scale, label):
    """out = (a/d*gamma + r) * scale, compared on the scale of the sum's two
    terms: (|a*gamma|/d + |r|) * |scale|."""
    a, r, g = f32(inp, "a"), f32(inp, "b"), f32(inp, "gamma")
    want, d = oracle.norm_then_add(a, r, g, inp["eps"], scale)
    sc = 1.0 if scale is None else abs(scale)
    den = (np.abs(a.astype(np.float64) * g) / d[:, None] + np.abs(r)) * sc
    err = scaled_error(out, want, den, NORMAL_MIN[inp["dtype"]])[0]
    tol = TOLS[inp["dtype"]]
    say(f"{label}: out err {err:.3e} (tol {tol:g}) shape {snr.last_shape()}")
    assert err <= tol, (label, err)


def check_add_norm(oracle, inp, s, y, label):
    """s compared on |a| + |b|, y on |gamma| (|a| + |b|) / d."""
    a, b, g = f32(inp, "a"), f32(inp, "b"), f32(inp, "gamma")
    ws, wy, d = oracle.add_then_norm(a, b, g, inp["eps"])
    den = np.abs(a.astype(np.float64)) + np.abs(b)
    fl = NORMAL_MIN[inp["dtype"]]
    es = scaled_error(s, ws, den, fl)[0]
    ey = scaled_error(y, wy, np.abs(g.astype(np.float64)) * den /
                      d[:, None], fl)[0]
    tol = TOLS[inp["dtype"]]
    say(f"{label}: sum err {es:.3e} y err {ey:.3e} (tol {tol:g}) shape "
        f"{snr.last_shape()}")
    assert es <= tol and ey <= tol, (label, es, ey)


def run_plain(inp, prefill=float("nan"), out_is_x=False):
    st = inp["dtype"]
    x, g = dev(inp["x"], st), dev(inp["gamma"], st)
    out = x if out_is_x else torch.full_like(x, prefill)
    snr.rmsnorm_fwd(x, g, inp["eps"], out=out)
    torch.cuda.synchronize()
    return host_f64(out), out


def run_tail(inp, prefill=float("nan"), in_place=False):
    st = inp["dtype"]
    a, r = dev(inp["a"], st), dev(inp["r"], st)
    gp, gq = dev(inp["gamma_post"], st), dev(inp["gamma_pre"], st)
    y = torch.full_like(a, prefill)
    if in_place:
        snr.sandwich_tail_inplace(a, r, gp, inp["eps_post"], gq,
                                  inp["eps_pre"], y_out=y)
        h = r
    else:
        h = torch.full_like(a, prefill)
        snr.sandwich_tail(a, r, gp, inp["eps_post"], gq, inp["eps_pre"],
                          h_out=h, y_out=y)
    torch.cuda.synchronize()
    return host_f64(h), host_f64(y)


def run_norm_add(inp, scale=None, in_place=False, prefill=float("nan")):
    st = inp["dtype"]
    a, r, g = dev(inp["a"], st), dev(inp["b"], st), dev(inp["gamma"], st)
    sc = None if scale is None else torch.tensor([scale], device=DEV)
    out = r if in_place else torch.full_like(a, prefill)
    snr.norm_then_add(a, r, g, inp["eps"], out_scale=sc, out=out)
    torch.cuda.synchronize()
    return host_f64(out)


def run_add_norm(inp, sum_into=None, prefill=float("nan")):
    """sum_into: None (fresh output), "a" or "b" (accumulate in place)."""
    st = inp["dtype"]
    a, b, g = dev(inp["a"], st), dev(inp["b"], st), dev(inp["gamma"], st)
    s = {"a": a, "b": b}.get(sum_into) if sum_into else \
        torch.full_like(a, prefill)
    y = torch.full_like(a, prefill)
    snr.add_then_norm(a, b, g, inp["eps"], sum_out=s, y_out=y)
    torch.cuda.synchronize()
    return host_f64(s), host_f64(y)


# -- RMSNorm into Q8_1 records ---------------------------------------------
# A code may differ from the oracle's by one only where the oracle's
# unrounded t = v / d lies within Q8_TIE of a rounding boundary k + 1/2: the
# GPU's t carries the f32 error of v and of d (a few units of 2^-24
# relative, so at most about 1e-4 absolute for |t| <= 127).
Q8_TIE = 1e-3


def run_q8(inp):
    """Q8_1 records of the inputs, as uint8 [rows, n / 32, 36] on the host."""
    st = inp["dtype"]
    x, g = dev(inp["x"], st), dev(inp["gamma"], st)
    out = snr.rmsnorm_q8_1(x, g, inp["eps"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_q8(oracle, inp, blocks, label):
    """Records against the oracle: s == 0; d within half an f16 unit of the
    oracle's scale (relative, measured against at least the smallest f16
    normal) plus f32 slack; zero blocks exactly zero; every code equal to
    the oracle's except next to a rounding tie, where it is one of the two
    neighbours. Returns (max relative d error, codes in the tie band)."""
    x, g = f32(inp, "x"), f32(inp, "gamma")
    _, d_o, t_o, q_o = oracle.rmsnorm_q8_1(x, g, inp["eps"])
    rows, n = x.shape
    assert blocks.shape == (rows, n // 32, 36) and blocks.dtype == np.uint8
    d = blocks[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    s = blocks[..., 2:4].copy().view(np.uint16)[..., 0]
    q = blocks[..., 4:36].copy().view(np.int8).reshape(rows, n)
    assert np.all(s == 0), label
    zero = d_o == 0
    assert np.all(d[zero] == 0), (label, "zero block with d != 0")
    derr = np.abs(d - d_o) / np.maximum(np.abs(d_o), 2.0 ** -14)
    worst_d = float(derr[~zero].max()) if np.any(~zero) else 0.0
    assert worst_d <= 2.0 ** -11 + 1e-5, (label, worst_d)
    frac = np.abs(np.abs(t_o) - np.floor(np.abs(t_o)) - 0.5)
    near = frac < Q8_TIE
    dq = q.astype(np.int64) - q_o.astype(np.int64)
    bad = (dq != 0) & ~near
    assert not np.any(bad), (label, int(bad.sum()), "codes differ")
    assert np.all(np.abs(dq[near]) <= 1), (label, "tie code off by > 1")
    say(f"{label}: d err {worst_d:.3e}, {int(near.sum())} codes of "
        f"{q.size} in the tie band, {int((dq != 0).sum())} differ; shape "
        f"{snr.last_shape()}")
    return worst_d, int(near.sum())
