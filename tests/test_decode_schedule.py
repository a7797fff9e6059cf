"""Host check of the decode kernel's share schedule (decode_schedule.h):
shares tile the unit list contiguously, share_of inverts the ranges, static
shares have the stated size and the share count stays within what the
workspace holds.  Compiled with g++ from the same header the kernel uses."""
import os
import random
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_110_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "schedule_check.cpp")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("sched") / "schedule_check")
    subprocess.run([gxx, "-O2", "-std=c++17", "-I", CSRC, SRC, "-o", exe], check=True)
    return exe


def _run(exe, pairs):
    text = "".join(f"{t} {w}\n" for t, w in pairs)
    res = subprocess.run([exe], input=text, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok")


def test_edge_sizes(checker):
    pairs = []
    for W in (1, 2, 7, 256, 2048, 4096, 8192):
        for T in (0, 1, 2, 31, 32, 33, 32 * W - 1, 32 * W, 32 * W + 1, 43 * W + 5,
                  100 * W, 100 * W + W // 2 + 3):
            pairs.append((T, W))
    _run(checker, pairs)


def test_workload_sizes(checker):
    # unit counts of the decode workloads (sequences x KV heads x 16-token tiles)
    pairs = [(141_000, 2048), (315_000, 2048), (517_000, 2048), (4, 2048), (2**31 - 1, 2048),
             (2**31 - 1, 1), (2**31 - 1, 8192)]
    _run(checker, pairs)


def test_random_sizes(checker):
    rng = random.Random(7)
    pairs = []
    for _ in range(300):
        W = rng.choice([1, 3, 64, 512, 1000, 2048, 4096])
        T = rng.choice([rng.randint(0, 64 * W), rng.randint(0, 10**6), rng.randint(0, 2**31 - 1)])
        pairs.append((T, W))
    _run(checker, pairs)
