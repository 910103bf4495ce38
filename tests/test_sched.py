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


# ---------------------------------------------------------------- decode cut

def decode_bounds(exe, n_wg, piece_cost, lens):
    out = subprocess.run([exe, "decode"], input=f"{n_wg} {piece_cost} {len(lens)} " + " ".join(map(str, lens)),
                         capture_output=True, text=True, check=True).stdout.split()
    return [int(x) for x in out]


def share_costs(bnd, lens, piece_cost):
    """Each share's pages plus piece_cost per segment it intersects (direct
    interval count)."""
    starts = np.concatenate([[0], np.cumsum(lens)])
    costs = []
    for a, b in zip(bnd, bnd[1:]):
        pieces = sum(1 for i in range(len(lens)) if starts[i] < b and starts[i + 1] > a)
        costs.append((b - a) + piece_cost * pieces)
    return costs


def decode_32k_lens():
    # 31 sequences of 32,769 keys on 64-key pages: 1 global head (513 pages), 7 local (W 4096: 65 pages)
    return [513] + [65] * 7


@pytest.mark.parametrize("n_wg,piece_cost,lens", [
    (256, 1, decode_32k_lens() * 31),
    (256, 0, decode_32k_lens() * 31),
    (7, 2, [5, 1, 1, 30, 2, 2, 9]),
    (3, 4, [100]),                                   # one segment, more shares than pieces needed
    (40, 1, list(np.random.default_rng(3).integers(1, 300, 500))),
    (1, 1, [4, 4]),
])
def test_decode_shares_cover_the_list_in_order(driver, n_wg, piece_cost, lens):
    bnd = decode_bounds(driver, n_wg, piece_cost, lens)
    assert len(bnd) == n_wg + 1 and bnd[0] == 0 and bnd[-1] == sum(lens)
    assert all(a <= b for a, b in zip(bnd, bnd[1:]))
    if piece_cost == 0:
        assert bnd == [sum(lens) * w // n_wg for w in range(n_wg + 1)]


@pytest.mark.parametrize("n_wg,lens", [
    (256, decode_32k_lens() * 31),
    (40, list(np.random.default_rng(3).integers(1, 300, 500))),
    (100, list(np.random.default_rng(4).integers(50, 600, 60))),
])
def test_decode_shares_even_out_piece_costs(driver, n_wg, lens):
    """With a piece cost, the dearest share costs less than with equal page
    counts, and no share is more than two pieces' cost above the mean."""
    c = 1
    even = share_costs(decode_bounds(driver, n_wg, 0, lens), lens, c)
    cut = share_costs(decode_bounds(driver, n_wg, c, lens), lens, c)
    assert max(cut) <= max(even)
    assert max(cut) <= np.mean(cut) + 2 * c + 1
