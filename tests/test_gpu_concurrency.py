"""Host threads calling the library at once, each on a stream of its own:
the tail, the plain norm and a split-row norm (the one path with a per-stream
workspace) give, bit for bit, what the same calls give alone, and no
split-row wait gives up. The library's per-call state (forced shape, last
shape, last HIP error) is per thread and its workspace is per (device,
stream); this checks both under concurrent use."""
import threading

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import dev, say  # noqa: E402

pytestmark = pytest.mark.gpu

THREADS = 4
REPEATS = 10
SPLIT_N = 2 * 65536        # 16 chunks of 2048 vectors: the split-row kernel


def _inputs(t):
    tail = gen.random_tail(64, 6656, 50000 + t)
    plain = gen.random_plain(64, 4099, 51000 + t)
    wide = gen.random_plain(8, SPLIT_N, 52000 + t)
    return {
        "tail": [dev(tail[k], "f32") for k in ("a", "r", "gamma_post",
                                               "gamma_pre")],
        "plain": [dev(plain[k], "f32") for k in ("x", "gamma")],
        "wide": [dev(wide[k], "f32") for k in ("x", "gamma")],
    }


def _run(d):
    """The three calls on the current stream; returns their outputs."""
    a, r, gp, gq = d["tail"]
    h, y = snr.sandwich_tail(a, r, gp, 1e-8, gq, 1e-5)
    x, g = d["plain"]
    p = snr.rmsnorm_fwd(x, g, 1e-5)
    wx, wg = d["wide"]
    with snr.forced_shape("split", 0, 8):
        w = snr.rmsnorm_fwd(wx, wg, 1e-5)
        shape = snr.last_shape()
    assert shape.startswith("split:"), shape
    return [h, y, p, w]


def test_threads_on_their_own_streams():
    say(f"{THREADS} threads x {REPEATS} repeats, own streams")
    data = [_inputs(t) for t in range(THREADS)]
    alone = []
    for d in data:
        outs = _run(d)
        torch.cuda.synchronize()
        alone.append([o.clone() for o in outs])

    streams = [torch.cuda.Stream() for _ in range(THREADS)]   # default priority
    results = [None] * THREADS
    errors = []
    start = threading.Barrier(THREADS)

    def worker(t):
        try:
            with torch.cuda.stream(streams[t]):
                start.wait()
                outs = None
                for _ in range(REPEATS):
                    outs = _run(data[t])
                streams[t].synchronize()
                results[t] = [o.clone() for o in outs]
                streams[t].synchronize()
                results[t].append(snr.split_timeouts(streams[t]))
        except Exception as e:  # reported below, in the test's thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,))
               for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker did not finish"
    assert not errors, errors
    for t in range(THREADS):
        *outs, timeouts = results[t]
        assert timeouts == 0, (t, timeouts)
        for got, want in zip(outs, alone[t]):
            assert torch.equal(got, want), t
    assert np.isfinite(alone[0][3].cpu().numpy()).all()
