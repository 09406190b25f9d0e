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
