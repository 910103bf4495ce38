"""Algorithmic work ledger of segmented attention (closed forms).

TEST INFRASTRUCTURE (see the package docstring of ``oracle``).

The pages count savings in arithmetic only and leave memory traffic and
launch cost out of that ledger ("RedKnot: Head-Aware KV Reuse and
SegPagedAttention" page, section "Performance Targets and the DeepSeek V4
Flash Benchmark").  Here:

* prefill work = 4 * D FLOPs per visible (query head, query, key) pair: one
  multiply-add per channel for the score and one per channel for the
  weighted value;
* decode traffic = every visible K and V row read once per (sequence, KV
  head), plus the query and output rows.
"""

from __future__ import annotations


def visible_count(p: int, window: int) -> int:
    """|{j : j <= p and (window == 0 or p - j < window)}| for a query at p >= 0."""
    return p + 1 if window == 0 else min(p + 1, window)


def visible_pairs(kv_len: int, q_len: int, window: int) -> int:
    """Sum of visible keys over the last q_len queries of a kv_len sequence.

    Closed form: sum over p in [a, kv_len) of min(p + 1, W) (p + 1 when
    global), with a = kv_len - q_len, split at p = W - 1.
    """
    a = kv_len - q_len
    if q_len <= 0:
        return 0

    def tri(n):  # 1 + 2 + ... + n
        return n * (n + 1) // 2

    if window == 0:
        return tri(kv_len) - tri(a)
    # positions with p + 1 <= W: p in [a, min(kv_len, W))
    growing_hi = min(kv_len, window)
    growing = tri(growing_hi) - tri(a) if growing_hi > a else 0
    flat = (kv_len - max(a, window)) * window if kv_len > max(a, window) else 0
    return growing + flat


def prefill_visible_flops(kv_lens, q_lens, windows, num_q_heads, head_dim) -> int:
    hkv = len(windows)
    group = num_q_heads // hkv
    pairs = 0
    for kv, q in zip(kv_lens, q_lens):
        for w in windows:
            pairs += group * visible_pairs(kv, q, w)
    return 4 * head_dim * pairs


def decode_visible_bytes(kv_lens, windows, num_q_heads, head_dim, elem_bytes=2) -> dict:
    """Bytes a single-token decode step must move (one query per sequence)."""
    kv = 0
    for n in kv_lens:
        for w in windows:
            kv += 2 * visible_count(n - 1, w) * head_dim * elem_bytes
    n = len(kv_lens)
    q_o = n * num_q_heads * head_dim * elem_bytes * 2
    return {"kv": kv, "q_o": q_o, "total": kv + q_o}


def head_row_ceiling(reusable_layers: int, total_layers: int,
                     local_heads: int, total_heads: int) -> float:
    """Share of (layer, head) attention rows eligible for reuse: the
    reusable-layer share times the local-head share."""
    return (reusable_layers / total_layers) * (local_heads / total_heads)
