"""Host-side logic of bench.py (no GPU): the one-GPU contract and the input-copy rule the
timed legs follow so that no call finds its inputs in the memory-side cache."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from kv_block_top_amd import workloads as wl  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused_before_any_gpu_work(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, **env))
    assert r.returncode == 2
    assert "runs on one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("footprint", [1 << 10, 1 << 20, 100 << 20, 256 << 20, 302 << 20,
                                       546 << 20, 4 << 30])
def test_rotation_reads_twice_the_cache_between_reuses(footprint):
    n = bench.rotation_copies(footprint)
    # between two uses of one copy the other n - 1 copies are read: at least twice the
    # memory-side cache, and one copy fewer would not be
    assert (n - 1) * footprint >= 2 * bench.MALL_BYTES
    assert n == 2 or (n - 2) * footprint < 2 * bench.MALL_BYTES
    assert n >= 2


def test_mixed_workload_alternates_two_copies():
    w = wl.config(5)
    ab = bench.algorithmic_bytes(w)
    assert ab > bench.MALL_BYTES
    assert bench.rotation_copies(ab) == 2
