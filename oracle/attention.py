"""fp64 CPU oracle of head-classified segmented attention.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its binding) never calls it, and it shares no code with it.

What is computed (the method reaches exactly this result, only faster):

* Every (layer, KV head) carries a class from an offline classification:
  global heads attend to the full causal context, local heads only to a
  sliding window of recent tokens ("Xiaohongshu Open-Sources RedKnot" page,
  section "What Happened", item 1).
* SegPagedAttention stores, per (layer, head), only the tokens the head
  needs and runs every head through fused varlen attention without building
  an attention mask (same page and section, item 3; "RedKnot: Head-Aware KV
  Reuse and SegPagedAttention" page, section "The Three Core Mechanisms in
  Detail", third mechanism).  Skipping keys a head can never see does not
  change the softmax, so the result is plain masked softmax attention with a
  per-head visibility predicate.

Readings taken where the pages are silent:

* A local head with window W sees the W most recent tokens including the
  query's own: key j is visible to the query at absolute position p iff
  ``p - W < j <= p``.  W = 0 encodes a global head (``j <= p``).
* The window slides with each query.
* Queries sit at the end of their sequence: query t of a sequence with
  ``kv_len`` cached tokens and ``q_len`` queries has position
  ``kv_len - q_len + t`` (its own key is already in the cache).
* Query head h uses KV head ``h // (Hq // Hkv)`` (contiguous GQA groups).
* ``lse`` is the natural log of the sum of exp of the *scaled* scores.

Everything is float64 from the exact bfloat16 input values; nothing is
rounded on the way.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def is_visible(p: int, j: int, window: int) -> bool:
    """Scalar visibility predicate (the definition, used by brute force)."""
    if j < 0 or j > p:
        return False
    return window == 0 or p - j <= window - 1


def query_positions(kv_len: int, q_len: int) -> np.ndarray:
    """Absolute positions of the last ``q_len`` tokens of a ``kv_len`` cache."""
    if q_len > kv_len or q_len < 0:
        raise ValueError("need 0 <= q_len <= kv_len")
    return np.arange(kv_len - q_len, kv_len, dtype=np.int64)


def visibility_mask(q_pos: np.ndarray, kv_len: int, window: int) -> np.ndarray:
    """bool [len(q_pos), kv_len]: entry (i, j) says key j is visible to query i."""
    if window < 0:
        raise ValueError("window must be >= 0 (0 = global)")
    j = np.arange(kv_len, dtype=np.int64)[None, :]
    p = np.asarray(q_pos, dtype=np.int64)[:, None]
    mask = j <= p
    if window > 0:
        mask &= (p - j) <= (window - 1)
    return mask


def masked_softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                             mask: np.ndarray, scale: float):
    """One head: q [n, D], k/v [m, D], mask bool [n, m] -> (o [n, D], lse [n]).

    Rows with no visible key would be undefined; the callers' visibility
    always includes the query's own key, and this function refuses such rows.
    """
    if not np.all(mask.any(axis=1)):
        raise ValueError("every query row needs at least one visible key")
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)                       # exactly 0 where masked
    l = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(l))[:, 0]
    o = (e / l) @ v
    return o, lse


def attend_sequence(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    windows, scale: float, rows=None, row_block: int = 256):
    """Attention of one sequence.

    q: f64 [q_len, Hq, D] (the last q_len tokens' queries); k, v: f64
    [kv_len, Hkv, D]; ``windows[g]`` is KV head g's window (0 = global).
    ``rows`` optionally restricts the computed query rows (indices into
    q_len); the result then holds only those rows, in that order.

    Rows are processed in blocks of ``row_block``; for each block only the
    key columns that at least one row of the block can see are multiplied
    (a column masked for every row contributes exactly zero).
    Returns (o f64 [n_rows, Hq, D], lse f64 [n_rows, Hq]).
    """
    q_len, hq, d = q.shape
    kv_len, hkv, _ = k.shape
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    pos_all = query_positions(kv_len, q_len)
    rows = np.arange(q_len) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((len(rows), hq, d))
    lse = np.empty((len(rows), hq))
    for b0 in range(0, len(rows), row_block):
        r = rows[b0:b0 + row_block]
        pos = pos_all[r]
        for g in range(hkv):
            mask = visibility_mask(pos, kv_len, int(windows[g]))
            cols = np.nonzero(mask.any(axis=0))[0]
            lo, hi = int(cols[0]), int(cols[-1]) + 1
            mk = mask[:, lo:hi]
            kk = k[lo:hi, g, :]
            vv = v[lo:hi, g, :]
            for h in range(g * group, (g + 1) * group):
                oh, lh = masked_softmax_attention(q[r, h, :], kk, vv, mk, scale)
                o[b0:b0 + len(r), h, :] = oh
                lse[b0:b0 + len(r), h] = lh
    return o, lse


def attend_batch(q_bits, k_bits, v_bits, cu_q, cu_kv, windows, scale,
                 rows_per_seq=None):
    """Varlen batch on bf16 bit patterns; returns per-sequence (o, lse) lists.

    q_bits: uint16 [sum q][Hq][D]; k_bits, v_bits: uint16 [sum kv][Hkv][D];
    cu_q, cu_kv: prefix sums.  ``rows_per_seq[b]`` optionally picks rows.
    """
    outs = []
    for b in range(len(cu_q) - 1):
        q = bf16_bits_to_f64(q_bits[cu_q[b]:cu_q[b + 1]])
        k = bf16_bits_to_f64(k_bits[cu_kv[b]:cu_kv[b + 1]])
        v = bf16_bits_to_f64(v_bits[cu_kv[b]:cu_kv[b + 1]])
        rows = None if rows_per_seq is None else rows_per_seq[b]
        if q.shape[0] == 0:
            outs.append((np.zeros((0,) + q.shape[1:]), np.zeros((0, q.shape[1]))))
            continue
        outs.append(attend_sequence(q, k, v, windows, scale, rows=rows))
    return outs


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Combine attention over disjoint key subsets into attention over their union.

    o_parts [S, ..., D] are each part's normalised outputs, lse_parts [S, ...]
    their log-sum-exps (-inf for a part with no visible key, which then gets
    weight zero).  lse = ln sum_s exp(lse_s); o = sum_s exp(lse_s - lse) o_s.
    This is the split-KV decode's final step.
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    if np.any(np.isneginf(m)):
        raise ValueError("at least one part must hold a visible key")
    w = np.exp(lse_parts - m)               # 0 for empty parts
    tot = w.sum(axis=0)
    lse = m + np.log(tot)
    o = np.einsum("s...,s...d->...d", w / tot, np.asarray(o_parts, dtype=np.float64))
    return o, lse


def paged_store(rows: np.ndarray, page_size: int, seed: int):
    """Store logical rows [n, ...] in pages placed at a seeded random
    physical order.  Returns (pool [n_pages, page_size, ...], page_table):
    logical page i sits at pool[page_table[i]]; unused slots are zero."""
    n = rows.shape[0]
    n_pages = -(-n // page_size)
    table = np.random.default_rng(seed).permutation(n_pages)
    pool = np.zeros((n_pages, page_size) + rows.shape[1:], dtype=rows.dtype)
    for i in range(n_pages):
        chunk = rows[i * page_size:(i + 1) * page_size]
        pool[table[i], :len(chunk)] = chunk
    return pool, table


def paged_gather(pool: np.ndarray, table, n: int) -> np.ndarray:
    """Read logical rows 0 .. n-1 back through a page table: row t is slot
    t % page_size of physical page table[t // page_size]."""
    page_size = pool.shape[1]
    out = np.empty((n,) + pool.shape[2:], dtype=pool.dtype)
    for t in range(n):
        out[t] = pool[table[t // page_size], t % page_size]
    return out


def paged_round_trip(k: np.ndarray, page_size: int, seed: int):
    """``paged_store`` then ``paged_gather``: returns (gathered rows, page_table).
    Used to show the oracle's result does not depend on physical page placement."""
    pool, table = paged_store(k, page_size, seed)
    return paged_gather(pool, table, k.shape[0]), table
