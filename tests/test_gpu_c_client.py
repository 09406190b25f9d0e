"""The C ABI called from a plain C program (tests/c_client/snr_client.c,
built by __graft_entry__.build() with gcc): nothing but libsnr and the HIP
runtime in the calling process, no PyTorch. Inputs come from the seeded
generator, and outputs are compared with the oracle here, so the program
checks the boundary as a C caller meets it: f32 tail, plain norm, in-place
tail, error codes of rejected calls, and a stream of the caller's own."""
import os
import subprocess

import numpy as np
import pytest

from sandwich_norm_residual_amd import inputs as gen
from parity import TOL_F32, plain_error, tail_errors

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client",
                      "snr_client")


def _write(path, arr):
    np.ascontiguousarray(arr, dtype=np.float32).tofile(path)


def _read(path, rows, n):
    return np.fromfile(path, dtype=np.float32).reshape(rows, n)


@pytest.mark.gpu
@pytest.mark.parametrize("rows,n", [(3, 6657), (64, 6656), (5, 2),
                                    (2, 65536 + 3)])
def test_c_client_matches_the_oracle(oracle, tmp_path, rows, n):
    assert os.path.exists(CLIENT), (
        f"{CLIENT} is not built; run __graft_entry__.build()")
    inp = gen.random_tail(rows, n, seed=9100 + n % 97 + rows)
    for key, name in (("a", "a"), ("r", "r"), ("gamma_post", "gp"),
                      ("gamma_pre", "gq")):
        _write(tmp_path / f"{name}.f32", inp[key])
    _write(tmp_path / "eps.f32", [inp["eps_post"], inp["eps_pre"]])
    print(f"[gpu-case] C client rows={rows} n={n}", flush=True)
    run = subprocess.run([CLIENT, str(tmp_path), str(rows), str(n)],
                         capture_output=True, text=True, timeout=90)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (
        run.returncode, run.stdout, run.stderr)

    h = _read(tmp_path / "h.f32", rows, n)
    y = _read(tmp_path / "y.f32", rows, n)
    o = oracle.sandwich_tail(inp["a"], inp["r"], inp["gamma_post"],
                             inp["eps_post"], inp["gamma_pre"], inp["eps_pre"])
    eh, ey = tail_errors(h, y, o, inp["r"], inp["gamma_pre"])
    print(f"[gpu-case] C client tail: h err {eh:.3e} y err {ey:.3e}",
          flush=True)
    assert eh <= TOL_F32 and ey <= TOL_F32, (eh, ey)

    z = _read(tmp_path / "z.f32", rows, n)
    want = oracle.rmsnorm(inp["a"], inp["gamma_post"], inp["eps_pre"])
    ez = plain_error(z, want)
    assert ez <= TOL_F32, ez

    # the in-place form runs the same kernel on the same shape
    hi = _read(tmp_path / "hi.f32", rows, n)
    yi = _read(tmp_path / "yi.f32", rows, n)
    assert np.array_equal(hi.view(np.uint32), h.view(np.uint32))
    assert np.array_equal(yi.view(np.uint32), y.view(np.uint32))
