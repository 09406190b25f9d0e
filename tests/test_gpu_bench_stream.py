"""The benchmark's streaming kernels (bench_stream.hip): each variant touches
exactly the bytes it is given, at every grid size bench.py uses, and the copy
copies. Buffers carry guard bands on both sides that must stay untouched."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "bench_stream.so")

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes on each side of the region
READ, WRITE, WRITE_NT, COPY = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    # PyTorch's HIP runtime first: this library names the same runtime
    # soname, and whichever copy a process loads first is the one it keeps.
    import torch
    torch.zeros(1, device="cuda:0")
    if not os.path.exists(PATH):
        pytest.fail(f"{PATH} is missing: run __graft_entry__.build()")
    L = ctypes.CDLL(PATH)
    L.stream_probe.restype = ctypes.c_int
    L.stream_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                               ctypes.c_void_p]
    return L


def _buffers(torch, nbytes):
    src = torch.randint(0, 256, (GUARD + nbytes + GUARD,), dtype=torch.uint8,
                        device="cuda:0")
    dst = torch.full((GUARD + nbytes + GUARD,), 0xA5, dtype=torch.uint8,
                     device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    return src, dst, sink


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000003])
@pytest.mark.parametrize("grid", [2048, 8192, 32768, 0, 1])
def test_variants_touch_exactly_their_bytes(lib, nbytes, grid):
    import torch
    print(f"bench_stream nbytes={nbytes} grid={grid}", flush=True)
    stream = torch.cuda.current_stream().cuda_stream
    for variant in (READ, WRITE, WRITE_NT, COPY):
        src, dst, sink = _buffers(torch, nbytes)
        before_src = src.clone()
        rc = lib.stream_probe(variant, src.data_ptr() + GUARD,
                              dst.data_ptr() + GUARD, sink.data_ptr(), nbytes,
                              grid, stream)
        assert rc == 0, (variant, rc)
        torch.cuda.synchronize()
        assert torch.equal(src, before_src), variant          # never written
        assert (dst[:GUARD] == 0xA5).all() and (dst[-GUARD:] == 0xA5).all()
        body = dst[GUARD:GUARD + nbytes]
        if variant == READ:
            assert (body == 0xA5).all()
            assert int(sink[0]) in (0, 0x9E3779B9 - (1 << 32))
        elif variant == COPY:
            assert torch.equal(body, src[GUARD:GUARD + nbytes])
        else:
            # the fill (lane, 1, 2, 3) as f32: every 16-byte vector's last
            # three words are 1.0, 2.0, 3.0
            words = body.view(torch.float32).view(-1, 4).cpu()
            assert (words[:, 1] == 1.0).all() and (words[:, 2] == 2.0).all()
            assert (words[:, 3] == 3.0).all()
            assert ((words[:, 0] >= 0) & (words[:, 0] < 256)).all()


def test_invalid_arguments_enqueue_nothing(lib):
    import torch
    src, dst, sink = _buffers(torch, 64)
    stream = torch.cuda.current_stream().cuda_stream
    p = src.data_ptr() + GUARD
    q = dst.data_ptr() + GUARD
    assert lib.stream_probe(COPY, p, q, sink.data_ptr(), 24, 0, stream) == -1
    assert lib.stream_probe(COPY, p + 4, q, sink.data_ptr(), 64, 0,
                            stream) == -1
    assert lib.stream_probe(7, p, q, sink.data_ptr(), 64, 0, stream) == -1
    torch.cuda.synchronize()
    assert (dst == 0xA5).all()


@pytest.mark.parametrize("two_in,two_out", [(True, True), (True, False),
                                            (False, False), (False, True)])
@pytest.mark.parametrize("lanes,vpt,nvec", [(1024, 2, 1664), (1024, 1, 1000),
                                            (512, 2, 832), (512, 4, 2048),
                                            (256, 2, 512), (256, 4, 7),
                                            (256, 8, 2048)])
def test_row_pattern_touches_exactly_its_rows(lib, lanes, vpt, nvec, two_in,
                                              two_out):
    """stream_probe_rows: h = a + r and y = a - r (r = a without a second
    input) on every vector of every row, nothing outside the [rows, nvec]
    regions, and no stream that was not passed is touched."""
    import torch
    lib.stream_probe_rows.restype = ctypes.c_int
    lib.stream_probe_rows.argtypes = [ctypes.c_void_p] * 4 + [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p]
    rows = 37
    print(f"bench_stream rows={rows} nvec={nvec} lanes={lanes} vpt={vpt} "
          f"two_in={two_in} two_out={two_out}", flush=True)
    g = GUARD // 4
    m = rows * nvec * 4
    a = torch.randn(g + m + g, device="cuda:0")
    r = torch.randn(g + m + g, device="cuda:0")
    h = torch.full((g + m + g,), 7.0, device="cuda:0")
    y = torch.full((g + m + g,), 7.0, device="cuda:0")
    a0, r0 = a.clone(), r.clone()
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.stream_probe_rows(a.data_ptr() + GUARD,
                               r.data_ptr() + GUARD if two_in else None,
                               h.data_ptr() + GUARD,
                               y.data_ptr() + GUARD if two_out else None,
                               rows, nvec, lanes, vpt, stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(a, a0) and torch.equal(r, r0)
    for t in (h, y):
        assert (t[:g] == 7.0).all() and (t[g + m:] == 7.0).all()
    body = slice(g, g + m)
    second = r[body] if two_in else a[body]
    assert torch.equal(h[body], a[body] + second)
    if two_out:
        assert torch.equal(y[body], a[body] - second)
    else:
        assert (y == 7.0).all()


def test_row_pattern_rejects_what_it_cannot_cover(lib):
    import torch
    lib.stream_probe_rows.restype = ctypes.c_int
    lib.stream_probe_rows.argtypes = [ctypes.c_void_p] * 4 + [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p]
    t = torch.zeros(4096, device="cuda:0")
    p = t.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.stream_probe_rows(p, p, p, p, 1, 2049, 1024, 2, stream) == -1
    assert lib.stream_probe_rows(p, p, p, p, 1, 64, 128, 2, stream) == -1
    assert lib.stream_probe_rows(p + 4, p, p, p, 1, 64, 256, 4, stream) == -1
    assert lib.stream_probe_rows(p, p, p, p, 0, 64, 256, 4, stream) == -1
    assert lib.stream_probe_rows(None, p, p, p, 1, 64, 256, 4, stream) == -1
    assert lib.stream_probe_rows(p, p, None, p, 1, 64, 256, 4, stream) == -1
    torch.cuda.synchronize()
    assert (t == 0).all()
