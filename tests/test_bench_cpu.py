"""bench.py's host logic, on the CPU: the algorithmic byte counts, the
committed rocprofv3 counter summaries (parseable, consistent with the byte
count, traffic close to it), and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sandwich_norm_residual_amd import inputs as gen  # noqa: E402

PROFILES = os.path.join(ROOT, "profiles")


def test_algorithmic_bytes_of_the_headline():
    # four row streams of 4096 x 6656 f32 and two gains
    assert bench.algorithmic_bytes(gen.CONFIGS["tail_4096x6656_f32"]) == \
        16 * 4096 * 6656 + 2 * 4 * 6656
    # Q8_1: x read, 36-byte records per 32 values written, gain once
    assert bench.algorithmic_bytes(gen.CONFIGS["q8_4096x6656_f32"]) == \
        4096 * 6656 * 4 + 6656 * 4 + 4096 * 6656 // 32 * 36


def _summaries():
    return sorted(f[:-len(".counters.txt")] for f in os.listdir(PROFILES)
                  if f.endswith(".counters.txt"))


@pytest.mark.parametrize("workload", _summaries())
def test_counter_summary_is_consistent(workload):
    kv = {}
    with open(os.path.join(PROFILES, f"{workload}.counters.txt")) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    cfg = gen.CONFIGS[workload]
    assert kv["workload"] == workload
    assert int(kv["algorithmic_bytes_per_launch"]) == \
        bench.algorithmic_bytes(cfg)
    traffic = float(kv["traffic_bytes_per_launch"])
    assert 0.98 <= traffic / bench.algorithmic_bytes(cfg) <= 1.05
    # the counters are scaled by a plain copy of known size
    assert abs(float(kv["fetch_scale"]) - 2.0) < 0.01
    assert abs(float(kv["write_scale"]) - 1.0) < 0.01
    assert os.path.exists(os.path.join(PROFILES,
                                       f"{workload}.kernel_trace.txt"))


def test_kernel_sources_by_kind():
    tail = [os.path.basename(p) for p in
            bench.kernel_sources(gen.CONFIGS["tail_4096x6656_f32"])]
    q8 = [os.path.basename(p) for p in
          bench.kernel_sources(gen.CONFIGS["q8_4096x6656_f32"])]
    assert "snr_kernels.hip" in tail and "snr_persist.hip" in tail
    assert "snr_q8.hip" in q8 and "snr_kernels.hip" not in q8
    for p in bench.kernel_sources(gen.CONFIGS["tail_4096x6656_f32"]):
        assert os.path.exists(p)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_graph_flag_is_parsed_before_the_gpu_check():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--graph", "--config", "tail_1x6656_f32", "--gpus",
                        "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_capture_steps_runs_each_step_twice_in_order():
    """capture_steps: one eager pass on a side stream, then the same steps
    under capture (torch's graph API replaced by a recorder)."""
    calls = []

    class _Ctx:
        def __init__(self, tag):
            self.tag = tag

        def __enter__(self):
            calls.append(("enter", self.tag))

        def __exit__(self, *exc):
            calls.append(("exit", self.tag))

    class _Stream:
        def wait_stream(self, other):
            pass

    class _Cuda:
        Stream = _Stream

        @staticmethod
        def current_stream():
            return _Stream()

        @staticmethod
        def stream(s):
            return _Ctx("side")

        @staticmethod
        def synchronize():
            pass

        class CUDAGraph:
            pass

        @staticmethod
        def graph(g):
            return _Ctx("capture")

    class _Torch:
        cuda = _Cuda

    g = bench.capture_steps(lambda i: calls.append(i), 3, _Torch)
    assert isinstance(g, _Cuda.CUDAGraph)
    assert calls == [("enter", "side"), 0, 1, 2, ("exit", "side"),
                     ("enter", "capture"), 0, 1, 2, ("exit", "capture")]


def test_read_write_split():
    cfgs = gen.CONFIGS
    # tail: a and r and both gains read; h and y written
    assert bench.read_write_bytes(cfgs["tail_4096x6656_f32"]) == \
        (8 * 4096 * 6656 + 2 * 4 * 6656, 8 * 4096 * 6656)
    # plain bf16: x and the gain read, y written
    assert bench.read_write_bytes(cfgs["plain_16384x4096_bf16"]) == \
        (2 * 16384 * 4096 + 2 * 4096, 2 * 16384 * 4096)
    # Q8_1: x and the gain read, records written
    assert bench.read_write_bytes(cfgs["q8_4096x6656_f32"]) == \
        (4 * 4096 * 6656 + 4 * 6656, 4096 * 6656 // 32 * 36)
    for name, cfg in cfgs.items():
        r, w = bench.read_write_bytes(cfg)
        assert r >= w > 0 and r + w == bench.algorithmic_bytes(cfg), name


def test_stream_probe_library_exports():
    """bench_stream.so (built by build()) loads without a GPU and exports its
    two entry points; the argument checks run before any HIP call."""
    import ctypes

    import torch  # noqa: F401  (its HIP runtime before the library's)
    path = os.path.join(ROOT, "bench_stream.so")
    if not os.path.exists(path):
        pytest.skip("bench_stream.so not built")
    lib = ctypes.CDLL(path)
    assert lib.stream_probe_variants() == 4
    lib.stream_probe.restype = ctypes.c_int
    lib.stream_probe.argtypes = [ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_int,
                                 ctypes.c_void_p]
    # invalid variant, size not a multiple of 16, null or misaligned buffers
    assert lib.stream_probe(4, 16, 16, 16, 16, 0, None) == -1
    assert lib.stream_probe(0, 16, 16, 16, 24, 0, None) == -1
    assert lib.stream_probe(0, None, 16, 16, 16, 0, None) == -1
    assert lib.stream_probe(3, 16, 8, 16, 16, 0, None) == -1
    assert lib.stream_probe(0, 16, None, None, 16, 0, None) == -1


def test_host_cpus_reports_the_affinity_mask(monkeypatch):
    """The CPU baseline's thread count is the affinity mask's CPU count,
    capped by OMP_NUM_THREADS when that states a smaller share, and the
    mask is reported as ranges."""
    monkeypatch.setattr(bench.os, "sched_getaffinity",
                        lambda pid: {0, 1, 2, 3, 8, 10, 11})
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    hw = bench.host_cpus()
    assert hw["affinity"] == 7 and hw["threads"] == 7
    assert hw["mask"] == "0-3,8,10-11"
    monkeypatch.setenv("OMP_NUM_THREADS", "4")
    assert bench.host_cpus()["threads"] == 4
    monkeypatch.setenv("OMP_NUM_THREADS", "64")
    assert bench.host_cpus()["threads"] == 7
