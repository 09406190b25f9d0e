"""A process whose very first library calls are made inside a HIP graph
capture: the per-device facts and the kernels' resident workgroup counts are
then queried during the capture (host queries only; nothing is enqueued by
them). Run in a fresh Python process so that nothing is cached yet; the
replays must equal eager calls made afterwards, bit for bit. The shapes
cover a row tile, a persistent tile and the choice between them by resident
counts (1024 rows of the 16-bit tail)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
import torch
sys.path.insert(0, ROOT)
import sandwich_norm_residual_amd as snr

dev = "cuda:0"
g = torch.Generator(device="cpu").manual_seed(5)
def rnd(*shape, dt=torch.float32):
    return torch.randn(*shape, generator=g).to(dt).to(dev)

cases = []
# bf16 tail, 1024 rows of 6656: chosen by resident counts
a, r = rnd(1024, 6656, dt=torch.bfloat16), rnd(1024, 6656, dt=torch.bfloat16)
gp, gq = rnd(6656, dt=torch.bfloat16), rnd(6656, dt=torch.bfloat16)
h, y = torch.empty_like(a), torch.empty_like(a)
cases.append((lambda: snr.sandwich_tail(a, r, gp, 1e-8, gq, 1e-5, h_out=h, y_out=y), [h, y]))
# f32 plain, 1024 rows of 16384: persistent 1024 x 4
x, gx = rnd(1024, 16384), rnd(16384)
yx = torch.empty_like(x)
cases.append((lambda: snr.rmsnorm_fwd(x, gx, 1e-5, out=yx), [yx]))
# f32 tail, 8 rows of 6656: row tile, gains loaded with the row
a2, r2, g2, q2 = rnd(8, 6656), rnd(8, 6656), rnd(6656), rnd(6656)
h2, y2 = torch.empty_like(a2), torch.empty_like(a2)
cases.append((lambda: snr.sandwich_tail(a2, r2, g2, 1e-8, q2, 1e-5, h_out=h2, y_out=y2), [h2, y2]))

graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):
    for call, _ in cases:
        call()
shapes = []
torch.cuda.synchronize()
for rep in range(3):
    for _, outs in cases:
        for o in outs:
            o.fill_(float("nan"))
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    got = [[o.clone() for o in outs] for _, outs in cases]
    for (call, outs), gl in zip(cases, got):
        call()
        torch.cuda.synchronize()
        shapes.append(snr.last_shape())
        for o, gv in zip(outs, gl):
            assert torch.equal(o.view(torch.int16) if o.dtype != torch.float32
                               else o.view(torch.int32),
                               gv.view(torch.int16) if gv.dtype != torch.float32
                               else gv.view(torch.int32)), (rep, shapes[-1])
print("first-call capture ok", sorted(set(shapes)), flush=True)
"""


def test_first_calls_inside_a_capture():
    print("[gpu-case] first library calls inside a graph capture "
          "(fresh process)", flush=True)
    code = "ROOT = " + repr(ROOT) + "\n" + SCRIPT
    proc = subprocess.run([sys.executable, "-c", code], cwd=ROOT,
                          capture_output=True, text=True, timeout=110)
    sys.stdout.write(proc.stdout[-2000:])
    sys.stderr.write(proc.stderr[-2000:])
    assert proc.returncode == 0, proc.returncode
    assert "first-call capture ok" in proc.stdout


NOALLOC_SCRIPT = r"""
import ctypes
import sys
import torch
sys.path.insert(0, ROOT)
import sandwich_norm_residual_amd as snr
from sandwich_norm_residual_amd import _lib

L = _lib.lib()
dev = "cuda:0"
g = torch.Generator(device="cpu").manual_seed(6)
rows, n = 12, 5 * 16384 + 7          # wider than any register tile: split rows
a, r = torch.randn(rows, n, generator=g).to(dev), torch.randn(rows, n, generator=g).to(dev)
gp = (1 + 0.1 * torch.randn(n, generator=g)).to(dev)
gq = (1 + 0.1 * torch.randn(n, generator=g)).to(dev)

def call(fn, h, y):
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = fn(p(a), p(r), p(gp), ctypes.c_float(1e-8), p(gq), ctypes.c_float(1e-5),
            p(h), p(y), ctypes.c_int64(rows), ctypes.c_int64(n),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, _lib.strerror(rc)

h, y = torch.empty_like(a), torch.empty_like(a)
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):        # the entry point's first call on the device
    call(L.sandwich_tail_noalloc, h, y)
assert snr.last_shape().startswith("split:"), snr.last_shape()
torch.cuda.synchronize()
h1, y1 = torch.empty_like(a), torch.empty_like(a)
h2, y2 = torch.empty_like(a), torch.empty_like(a)
for rep in range(3):
    h.fill_(float("nan")); y.fill_(float("nan"))
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    call(L.sandwich_tail_noalloc, h1, y1)     # eager: clears the array first
    call(L.sandwich_tail, h2, y2)
    torch.cuda.synchronize()
    for got in ((h, y), (h1, y1)):
        for o, w in zip(got, (h2, y2)):
            assert torch.equal(o.view(torch.int32), w.view(torch.int32)), rep
print("noalloc first-call capture ok", snr.split_timeouts(), flush=True)
"""


def test_noalloc_first_call_inside_a_capture():
    """The allocation-free tail's first call on a device recorded into a
    graph (its scratch array's address is looked up during the capture, and
    the clear waits for the first eager call): three replays and the eager
    calls after each equal sandwich_tail bit for bit (a wait that gave up
    would have left NaN rows), and sandwich_tail's own waits all
    completed."""
    print("[gpu-case] sandwich_tail_noalloc first called inside a graph "
          "capture (fresh process)", flush=True)
    code = "ROOT = " + repr(ROOT) + "\n" + NOALLOC_SCRIPT
    proc = subprocess.run([sys.executable, "-c", code], cwd=ROOT,
                          capture_output=True, text=True, timeout=110)
    sys.stdout.write(proc.stdout[-2000:])
    sys.stderr.write(proc.stderr[-2000:])
    assert proc.returncode == 0, proc.returncode
    last = [ln for ln in proc.stdout.splitlines()
            if ln.startswith("noalloc first-call capture ok")]
    assert last and last[0].split()[-1] == "0", proc.stdout[-500:]
