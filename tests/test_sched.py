"""The host's static balancing of prefill work items over workgroups
(segkv_sched.h), driven on the CPU: every item lands in exactly one
workgroup's range, ranges follow the greedy least-loaded rule, and the
ranges agree with the per-item assignment.  (A workgroup range that did not
match its items once sent a zero item, with no tiles, to the device.)"""

import heapq
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "long_context_serving_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    exe = str(tmp_path_factory.mktemp("sched") / "sched_check")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", CSRC, os.path.join(HERE, "sched_check.cpp"), "-o", exe],
                   check=True)
    return exe


def run(exe, n_bins, cost):
    out = subprocess.run([exe], input=f"{n_bins} {len(cost)} " + " ".join(map(str, cost)), capture_output=True,
                         text=True, check=True).stdout.split("\n")
    return [int(x) for x in out[0].split()], [int(x) for x in out[1].split()]


def greedy(n_bins, cost):
    """Least-loaded bin first, ties to the lowest index (a direct priority
    queue of (load, bin))."""
    h = [(0, b) for b in range(n_bins)]
    owner = []
    for c in cost:
        load, b = heapq.heappop(h)
        owner.append(b)
        heapq.heappush(h, (load + c, b))
    return owner


@pytest.mark.parametrize("n_bins,cost", [
    (8, [10, 7, 7, 7, 6, 6, 6, 6]),          # one item per workgroup
    (4, [9, 9, 3, 3, 3, 3, 3, 1, 1]),
    (3, [5]),                                  # fewer items than workgroups
    (256, list(np.random.default_rng(1).integers(3, 300, 5000))),
    (7, list(np.random.default_rng(2).integers(1, 20, 200))),
])
def test_ranges_match_greedy_assignment(driver, n_bins, cost):
    off, order = run(driver, n_bins, cost)
    assert len(off) == n_bins + 1 and off[0] == 0 and off[-1] == len(cost)
    assert all(a <= b for a, b in zip(off, off[1:]))
    assert sorted(order) == list(range(len(cost)))
    owner = greedy(n_bins, cost)
    for b in range(n_bins):
        got = order[off[b]:off[b + 1]]
        assert got == [i for i in range(len(cost)) if owner[i] == b]
    if len(cost) >= n_bins:
        assert all(off[b + 1] > off[b] for b in range(n_bins)), "a workgroup was left without items"
