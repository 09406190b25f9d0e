"""The split-row kernels' cross-workgroup protocol and their workspaces, on
the GPU: a wait that gives up leaves nothing a later call could take for its
own (no count read in between), the wrap of the launch tags, calls on more
streams than there are workspaces (bounded device memory, every result
checked against the oracle), and HIP-graph capture of split-row and
multi-pass calls (replays bit for bit against eager; a stream without a
workspace is refused under capture)."""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import _lib  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import (DEV, check_plain, check_tail, dev, host_f64,  # noqa: E402
                         run_plain, run_tail, say)

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_gave_up_wait_does_not_leak_into_the_next_call(oracle, monkeypatch):
    """A call whose waits all give up (a budget of no polls; every kernel
    still exits) writes NaN to every output of its rows, so the failure is
    visible, and leaves published slots behind. The next call, made without
    reading or clearing the overrun count, must still match the oracle: its
    tag differs from every slot left behind."""
    for op, rows, n in (("plain", 48, 9 * 4096 + 3), ("tail", 40, 7 * 4096)):
        say(f"gave-up wait then normal call: {op} rows={rows} n={n}")
        with snr.forced_shape("split"):
            monkeypatch.setenv("SNR_SPLIT_SPIN_LIMIT", "0")
            if op == "plain":
                bad, _ = run_plain(gen.random_plain(rows + 8, n, 6100))
                assert np.isnan(bad).all()
            else:
                bh, by = run_tail(gen.random_tail(rows + 8, n, 6101))
                assert np.isnan(bh).all() and np.isnan(by).all()
            monkeypatch.delenv("SNR_SPLIT_SPIN_LIMIT")
            if op == "plain":
                inp = gen.random_plain(rows, n, 6102)
                got, _ = run_plain(inp)
                check_plain(oracle, inp, got, f"after-gave-up-{op}")
            else:
                inp = gen.random_tail(rows, n, 6103)
                h, y = run_tail(inp)
                check_tail(oracle, inp, h, y, f"after-gave-up-{op}")
            shape = snr.last_shape()
        assert shape.startswith("split:"), shape
        # the first call's overruns were counted; reading clears the count
        assert snr.split_timeouts() > 0
        assert snr.split_timeouts() == 0


_WRAP_CHILD = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r})
    sys.path.insert(0, {tests!r})
    import numpy as np
    import torch
    import oracle
    import sandwich_norm_residual_amd as snr
    from sandwich_norm_residual_amd import inputs as gen
    from gpu_helpers import run_plain, run_tail
    from parity import plain_error, tail_errors
    O = oracle.load()
    worst = 0.0
    # tags 2^31 - 2, 2^31 - 1, then (the slots cleared, the tags wrapped)
    # 1, 2, ...: rows and widths vary so that later launches leave earlier
    # launches' slots untouched
    shapes = [(30, 6 * 4096 + 1), (50, 9 * 4096), (12, 6 * 4096 + 1),
              (50, 9 * 4096), (7, 3 * 4096 + 2)]
    with snr.forced_shape("split"):
        for i, (rows, n) in enumerate(shapes):
            print("[wrap] call", i, rows, n, flush=True)
            if i % 2 == 0:
                inp = gen.random_plain(rows, n, 6200 + i)
                got, _ = run_plain(inp)
                want = O.rmsnorm(inp["x"], inp["gamma"], inp["eps"])
                worst = max(worst, plain_error(got, want))
            else:
                inp = gen.random_tail(rows, n, 6200 + i)
                h, y = run_tail(inp)
                o = O.sandwich_tail(inp["a"], inp["r"], inp["gamma_post"],
                                    inp["eps_post"], inp["gamma_pre"],
                                    inp["eps_pre"])
                worst = max(worst, *tail_errors(h, y, o, inp["r"],
                                                 inp["gamma_pre"]))
            assert snr.last_shape().startswith("split:"), snr.last_shape()
    print("[wrap] worst", worst, "timeouts", snr.split_timeouts(), flush=True)
""")


def test_launch_tags_wrap():
    """A fresh process whose first workspace starts its tags two launches
    before they wrap (SNR_SPLIT_EPOCH): five split-row calls across the wrap
    all match the oracle and no wait gives up."""
    say("launch tag wrap (child process)")
    env = dict(os.environ)
    env["SNR_SPLIT_EPOCH"] = str(2 ** 31 - 3)
    code = _WRAP_CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    r = subprocess.run([sys.executable, "-c", code], env=env,
                       capture_output=True, text=True, timeout=300)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0, r.stderr[-2000:]
    last = [ln for ln in r.stdout.splitlines() if ln.startswith("[wrap] worst")]
    assert last, r.stdout
    _, _, worst, _, timeouts = last[0].split()
    assert float(worst) <= 1e-5
    assert int(timeouts) == 0


def test_more_streams_than_workspaces(oracle):
    """Split-row calls on twelve streams, launched back to back without
    synchronising (eight workspaces per device: streams take workspaces over
    and wait on the GPU for their last use). Every result matches the
    oracle, and the library's device memory stays within 8 MiB."""
    nstreams, rows, n = 12, 24, 5 * 4096 + 1
    say(f"{nstreams} streams, split rows={rows} n={n}")
    inps = [gen.random_plain(rows, n, 6300 + i) for i in range(nstreams)]
    xs = [dev(i["x"], "f32") for i in inps]
    gs = [dev(i["gamma"], "f32") for i in inps]
    ys = [torch.full_like(x, float("nan")) for x in xs]
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    # the runtime's own per-stream resources come with a stream's first
    # work: give every stream some before measuring
    for i in range(nstreams):
        with torch.cuda.stream(streams[i]):
            ys[i].fill_(float("nan"))
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    with snr.forced_shape("split"):
        for rep in range(3):
            for i in range(nstreams):
                streams[i].wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(streams[i]):
                    snr.rmsnorm_fwd(xs[i], gs[i], inps[i]["eps"], out=ys[i])
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    say(f"device memory taken by the library: {(free0 - free1) / 2**20:.2f} "
        f"MiB")
    assert free0 - free1 <= 8 * 2 ** 20 + 2 ** 20
    for i in range(nstreams):
        check_plain(oracle, inps[i], host_f64(ys[i]), f"stream-{i}")
        assert snr.split_timeouts(streams[i]) == 0


def _graph_case(kind, op):
    rows, n = (9, 5 * 4096 + 3) if kind == "split" else (5, 3 * 16384 + 3)
    if op == "plain":
        inp = gen.random_plain(rows, n, 6400)
        ins = [dev(inp["x"], "f32"), dev(inp["gamma"], "f32")]

        def call(outs):
            snr.rmsnorm_fwd(ins[0], ins[1], inp["eps"], out=outs[0])
        nout = 1
    else:
        inp = gen.random_tail(rows, n, 6401)
        ins = [dev(inp[k], "f32")
               for k in ("a", "r", "gamma_post", "gamma_pre")]

        def call(outs):
            snr.sandwich_tail(ins[0], ins[1], ins[2], inp["eps_post"], ins[3],
                              inp["eps_pre"], h_out=outs[0], y_out=outs[1])
        nout = 2
    outs = [torch.empty_like(ins[0]) for _ in range(nout)]
    return inp, ins, call, outs


@pytest.mark.parametrize("kind", ["split", "multipass"])
@pytest.mark.parametrize("op", ["plain", "tail"])
def test_graph_capture_replays_match_eager(oracle, kind, op):
    """A wide-row call recorded into a HIP graph on a stream that already
    holds a workspace: four replays, with eager work and synchronisations
    between them and the outputs poisoned, each bit for bit equal to the
    eager call (and that equal to the oracle)."""
    say(f"graph capture {kind} {op}")
    inp, ins, call, outs = _graph_case(kind, op)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with snr.forced_shape(kind):
        with torch.cuda.stream(s):
            call(outs)          # the stream's workspace, outside the capture
        s.synchronize()
        shape = snr.last_shape()
        assert shape.startswith(kind + ":"), shape
        want = [o.clone() for o in outs]
        g = torch.cuda.CUDAGraph()
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            call(outs)
    torch.cuda.synchronize()
    if op == "plain":
        check_plain(oracle, inp, host_f64(want[0]), f"graph-{kind}-eager")
    else:
        check_tail(oracle, inp, host_f64(want[0]), host_f64(want[1]),
                   f"graph-{kind}-eager")
    for replay in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        for w, o in zip(want, outs):
            assert torch.equal(w, o), (kind, op, replay)
        say(f"graph {kind} {op}: replay {replay} matches eager")
    assert snr.split_timeouts(s) == 0


def test_capture_without_a_workspace_is_refused():
    """Under capture, a stream that holds no workspace cannot get one: the
    call returns SNR_ERR_CAPTURE and enqueues nothing."""
    say("capture without a workspace")
    inp = gen.random_plain(3, 5 * 4096, 6500)
    x, gm = dev(inp["x"], "f32"), dev(inp["gamma"], "f32")
    y = torch.empty_like(x)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with snr.forced_shape("split"):
        with torch.cuda.graph(g, stream=s):
            with pytest.raises(_lib.SnrError) as e:
                snr.rmsnorm_fwd(x, gm, inp["eps"], out=y)
    assert e.value.code == _lib.SNR_ERR_CAPTURE


def test_release_workspaces(oracle):
    """snr_release_workspaces frees the device's workspaces after their last
    uses: split-row calls on three streams, released and made again five
    times, match the oracle every time, and the device memory in use does
    not grow over the cycles. (The runtime carves 1 MiB allocations out of
    larger blocks and may keep freed ones, so free memory is not a count of
    workspaces.) A workspace recorded into a graph is kept: its graph still
    replays bit for bit after a release."""
    rows, n = 6, 4 * 4096 + 1
    inps = [gen.random_plain(rows, n, 6600 + i) for i in range(3)]
    xs = [dev(i["x"], "f32") for i in inps]
    gs = [dev(i["gamma"], "f32") for i in inps]
    ys = [torch.full_like(x, float("nan")) for x in xs]
    streams = [torch.cuda.Stream() for _ in range(3)]
    for i in range(3):
        with torch.cuda.stream(streams[i]):
            ys[i].fill_(float("nan"))
    torch.cuda.synchronize()

    def calls(label):
        with snr.forced_shape("split"):
            for i in range(3):
                streams[i].wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(streams[i]):
                    snr.rmsnorm_fwd(xs[i], gs[i], inps[i]["eps"], out=ys[i])
        torch.cuda.synchronize()
        for i in range(3):
            assert snr.split_timeouts(streams[i]) == 0
            check_plain(oracle, inps[i], host_f64(ys[i]), f"{label}-{i}")
            ys[i].fill_(float("nan"))
        torch.cuda.synchronize()

    used = []
    for cycle in range(6):
        calls(f"release-cycle{cycle}")
        snr.release_workspaces()
        free, total = torch.cuda.mem_get_info()
        used.append(total - free)
    say("device memory in use after each release (MiB): " +
        " ".join(f"{(u - used[0]) / 2**20:+.1f}" for u in used))
    assert max(used[1:]) <= used[0] + 2 ** 20

    # a workspace recorded into a graph stays through a release
    s = streams[0]
    with snr.forced_shape("split"):
        with torch.cuda.stream(s):
            snr.rmsnorm_fwd(xs[0], gs[0], inps[0]["eps"], out=ys[0])
        s.synchronize()
        want = ys[0].clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            snr.rmsnorm_fwd(xs[0], gs[0], inps[0]["eps"], out=ys[0])
    torch.cuda.synchronize()
    snr.release_workspaces()
    for replay in range(2):
        ys[0].fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        assert torch.equal(ys[0], want), replay
