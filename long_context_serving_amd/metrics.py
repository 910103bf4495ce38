"""Algorithmic work of a workload, for throughput reporting.

Counts only what the method must do: for prefill, 4 * D FLOPs per visible
(query head, query, key) pair (one multiply-add per channel for q.k and one
for p * v); for decode, every visible K and V row once per (sequence, KV
head) plus the query and output rows.  The compute ledger of the pages
likewise counts arithmetic and leaves memory traffic and launch cost out
("RedKnot: Head-Aware KV Reuse and SegPagedAttention" page, section
"Performance Targets and the DeepSeek V4 Flash Benchmark").
"""

from __future__ import annotations

import numpy as np

from .workloads import Workload


def visible_keys(positions: np.ndarray, window: int) -> np.ndarray:
    """Visible key count of each query position for one head class."""
    pos = np.asarray(positions, dtype=np.int64)
    return pos + 1 if window == 0 else np.minimum(pos + 1, window)


def prefill_flops(w: Workload, windows=None) -> int:
    windows = w.windows if windows is None else windows
    total = 0
    for kv, q in zip(w.kv_lens, w.q_lens):
        pos = np.arange(kv - q, kv, dtype=np.int64)
        for win in windows:
            total += int(visible_keys(pos, int(win)).sum()) * w.group
    return 4 * w.head_dim * total


def prefill_flops_rows(w: Workload, b: int, rows, windows=None) -> int:
    """FLOPs of selected query rows (indices into sequence b's queries)."""
    windows = w.windows if windows is None else windows
    pos = w.kv_lens[b] - w.q_lens[b] + np.asarray(rows, dtype=np.int64)
    return 4 * w.head_dim * w.group * sum(int(visible_keys(pos, int(win)).sum()) for win in windows)


def decode_bytes(w: Workload, windows=None, elem_bytes: int = 2) -> dict:
    windows = w.windows if windows is None else windows
    kv = 0
    for n in w.kv_lens:
        for win in windows:
            kv += 2 * int(visible_keys(np.array([n - 1]), int(win))[0]) * w.head_dim * elem_bytes
    q_o = 2 * w.n_seqs * w.num_q_heads * w.head_dim * elem_bytes
    return {"kv": kv, "q_o": q_o, "total": kv + q_o}


def merge_bytes(mode: np.ndarray, head_dim: int, elem_bytes: int = 2) -> dict:
    """Algorithmic HBM bytes of the head-decomposition merge: each (row,
    head) reads its mode byte and the partials its mode needs (o row and
    lse of A, of B, or of both) and writes one o row and one lse."""
    mode = np.asarray(mode)
    part = head_dim * elem_bytes + 4
    n_a = int(np.count_nonzero(mode == 0))
    n_b = int(np.count_nonzero(mode == 1))
    n_m = int(mode.size - n_a - n_b)
    read = mode.size + (n_a + n_b) * part + 2 * n_m * part
    write = mode.size * part
    return {"pairs": int(mode.size), "take_a": n_a, "take_b": n_b, "merge": n_m,
            "read": read, "write": write, "total": read + write}
