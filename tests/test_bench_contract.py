"""bench.py's contract on the CPU: one GPU only (N > 1 exits with a message before touching
a device), and the algorithmic byte counts the roofline divides by."""
import importlib.util
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes():
    b = _bench()

    class T:
        def __init__(self, shape):
            self.data = np.zeros(shape, np.uint16)  # bf16 bits

    class W:
        tensors = [T((2048, 4, 4096)), T((4096, 16384)), T((16384, 4096))]

    # 2 B read + 1 B written per bf16 element, plus 12 B per tensor (scale read, amax
    # read and write): 167,772,160 elements -> 503,316,480 + 36
    assert b.alg_bytes_quantize(W) == 3 * 167772160 + 36
    # history read + in-place write, amax read + reset write, scale read + write,
    # scale_inv write, one format byte per tensor
    n, H = 1152, 1024
    assert b.alg_bytes_update(n, H) == 2 * H * n * 4 + 8 * n + 8 * n + 4 * n + n == 9461376


def test_rejects_empty_timed_region():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--steps" in r.stderr and r.stdout == ""


def test_headline_is_the_largest_step():
    """The default workload is the hidden-12288 MLP's full step (5 tensors, 1.36 G
    elements): 4,076,863,488 algorithmic bytes plus 12 per tensor."""
    b = _bench()
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'default="mlp_12288"' in src

    class T:
        def __init__(self, n):
            self.data = np.lib.stride_tricks.as_strided(np.zeros(1, np.uint16), (n,), (0,))

    class W:
        tensors = [T(2048 * 12288), T(2048 * 49152), T(12288 * 49152), T(49152 * 12288),
                   T(2048 * 12288)]

    assert b.alg_bytes_quantize(W) == 4076863488 + 5 * 12


def test_cpu_baseline_uses_every_allowed_cpu():
    b = _bench()
    n = b.host_cpus()
    assert 1 <= n <= len(os.sched_getaffinity(0))
