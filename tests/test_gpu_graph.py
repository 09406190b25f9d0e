"""The row-tile and persistent kernels allocate nothing, synchronise nothing
and use no workspace, so a caller can record them into a HIP graph. Each
case captures one call on torch's capture stream, then replays the graph
several times with ordinary eager work and synchronisations between the
replays (outputs poisoned with NaN, inputs replaced), and checks every
replay bit for bit against the eager call on the same inputs."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sandwich_norm_residual_amd as snr  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402
from gpu_helpers import dev, say  # noqa: E402

pytestmark = pytest.mark.gpu


def _plain(st, rows, n):
    def setup(seed):
        inp = gen.random_plain(rows, n, seed, dtype=st)
        return [dev(inp["x"], st)], [dev(inp["gamma"], st)]

    def call(ins, gains, outs):
        snr.rmsnorm_fwd(ins[0], gains[0], 1e-5, out=outs[0])

    def outputs(ins):
        return [torch.empty_like(ins[0])]
    return setup, call, outputs


def _tail(st, rows, n):
    def setup(seed):
        inp = gen.random_tail(rows, n, seed, dtype=st)
        return ([dev(inp["a"], st), dev(inp["r"], st)],
                [dev(inp["gamma_post"], st), dev(inp["gamma_pre"], st)])

    def call(ins, gains, outs):
        snr.sandwich_tail(ins[0], ins[1], gains[0], 1e-8, gains[1], 1e-5,
                          h_out=outs[0], y_out=outs[1])

    def outputs(ins):
        return [torch.empty_like(ins[0]), torch.empty_like(ins[0])]
    return setup, call, outputs


def _norm_add(st, rows, n):
    def setup(seed):
        inp = gen.random_pair("norm_add", rows, n, seed, dtype=st)
        scale = torch.tensor([1.5], device="cuda:0")
        return ([dev(inp["a"], st), dev(inp["b"], st)],
                [dev(inp["gamma"], st), scale])

    def call(ins, gains, outs):
        snr.norm_then_add(ins[0], ins[1], gains[0], 1e-8, out_scale=gains[1],
                          out=outs[0])

    def outputs(ins):
        return [torch.empty_like(ins[0])]
    return setup, call, outputs


def _add_norm(st, rows, n):
    def setup(seed):
        inp = gen.random_pair("add_norm", rows, n, seed, dtype=st)
        return [dev(inp["a"], st), dev(inp["b"], st)], [dev(inp["gamma"], st)]

    def call(ins, gains, outs):
        snr.add_then_norm(ins[0], ins[1], gains[0], 1e-5, sum_out=outs[0],
                          y_out=outs[1])

    def outputs(ins):
        return [torch.empty_like(ins[0]), torch.empty_like(ins[0])]
    return setup, call, outputs


def _multi(st, rows, n):
    def setup(seed):
        a = gen.random_plain(rows, n, seed, dtype=st)
        b = gen.random_plain(rows // 4, n, seed + 1, dtype=st)
        return ([dev(a["x"], st), dev(b["x"], st)],
                [dev(a["gamma"], st), dev(b["gamma"], st)])

    def call(ins, gains, outs):
        snr.rmsnorm_fwd_multi([(ins[0], gains[0], 1e-5),
                               (ins[1], gains[1], 1e-6)], outs)

    def outputs(ins):
        return [torch.empty_like(t) for t in ins]
    return setup, call, outputs


def _q8(st, rows, n):
    def setup(seed):
        inp = gen.random_plain(rows, n, seed, dtype=st)
        return [dev(inp["x"], st)], [dev(inp["gamma"], st)]

    def call(ins, gains, outs):
        snr.rmsnorm_q8_1(ins[0], gains[0], 1e-5, out=outs[0])

    def outputs(ins):
        r, n_ = ins[0].shape
        return [torch.empty((r, n_ // 32, 36), dtype=torch.uint8,
                            device=ins[0].device)]
    return setup, call, outputs


CASES = {
    "plain-f32-64x6656": _plain("f32", 64, 6656),
    "plain-bf16-300x4096": _plain("bf16", 300, 4096),
    "plain-f16-1000x128": _plain("f16", 1000, 128),
    "tail-f32-8x6656": _tail("f32", 8, 6656),
    "tail-bf16-64x6657": _tail("bf16", 64, 6657),
    "norm_add-f32-33x4099": _norm_add("f32", 33, 4099),
    "add_norm-f16-21x2051": _add_norm("f16", 21, 2051),
    "multi-f32-416x128": _multi("f32", 416, 128),
    "q8-f32-600x6656": _q8("f32", 600, 6656),
    "q8-bf16-77x2560": _q8("bf16", 77, 2560),
}


def _poison(outs):
    for t in outs:
        if t.dtype == torch.uint8:
            t.fill_(0xA5)
        else:
            t.fill_(float("nan"))


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_eager(name):
    setup, call, outputs = CASES[name]
    say(f"graph {name}")
    ins, gains = setup(31000)
    outs = outputs(ins)
    # eager call first: any per-device state (occupancy queries) is set up
    # outside the capture
    call(ins, gains, outs)
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    _poison(outs)
    with torch.cuda.graph(g):
        call(ins, gains, outs)
    torch.cuda.synchronize()

    for replay in range(4):
        if replay == 2:
            # new inputs in the captured buffers: eager reference again
            new_ins, _ = setup(31000 + replay)
            for dst, src in zip(ins, new_ins):
                dst.copy_(src)
            ref = outputs(ins)
            call(ins, gains, ref)
            torch.cuda.synchronize()
            want = [t.clone() for t in ref]
        _poison(outs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for w, o in zip(want, outs):
            assert torch.equal(w.view(torch.uint8) if w.dtype != torch.uint8
                               else w,
                               o.view(torch.uint8) if o.dtype != torch.uint8
                               else o), (name, replay)
        say(f"graph {name}: replay {replay} matches eager")
