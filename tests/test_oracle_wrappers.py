"""Pins of the oracle's batch and row-subset wrappers.

The GPU parity tests at full size compare the kernels with
``attend_batch(..., rows_per_seq=...)`` (varlen slicing by cu_q / cu_kv, then
``attend_sequence(rows=...)``) and with ``attend_batch_relocated``.  These
tests pin those wrappers against the separately written brute force and
against the plain per-sequence call, on inputs chosen so that a plausible
slip (cu_q and cu_kv swapped, a sequence's rows taken from its neighbour,
rows returned sorted instead of in the order asked for, a block boundary
dropping a row, another sequence's relocation offset) fails at least one.
"""

import numpy as np
import pytest

from brute import brute_attention
from long_context_serving_amd import workloads as wl
from oracle import attention as A
from oracle import rope as RP


def _bits(rng, shape, scale=1.0):
    return wl.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def _varlen_batch(seed):
    """Three sequences with q_len != kv_len for two of them (one chunked),
    plus an empty query chunk, so cu_q and cu_kv differ everywhere."""
    rng = np.random.default_rng(seed)
    kv_lens = [13, 9, 11, 6]
    q_lens = [13, 4, 0, 1]
    hq, hkv, d = 4, 2, 6
    cu_kv = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int64)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    q = _bits(rng, (int(cu_q[-1]), hq, d), 1.5)
    k = _bits(rng, (int(cu_kv[-1]), hkv, d))
    v = _bits(rng, (int(cu_kv[-1]), hkv, d))
    return q, k, v, cu_q, cu_kv, kv_lens, q_lens


@pytest.mark.parametrize("windows", [(0, 3), (2, 0), (5, 5)])
def test_attend_batch_slices_each_sequence(windows):
    q, k, v, cu_q, cu_kv, kv_lens, q_lens = _varlen_batch(7)
    scale = 0.45
    outs = A.attend_batch(q, k, v, cu_q, cu_kv, windows, scale)
    assert len(outs) == len(kv_lens)
    for b, (o, lse) in enumerate(outs):
        assert o.shape[0] == q_lens[b] and lse.shape[0] == q_lens[b]
        if q_lens[b] == 0:
            continue
        qb = A.bf16_bits_to_f64(q[cu_q[b]:cu_q[b + 1]])
        kb = A.bf16_bits_to_f64(k[cu_kv[b]:cu_kv[b + 1]])
        vb = A.bf16_bits_to_f64(v[cu_kv[b]:cu_kv[b + 1]])
        ob, lb = brute_attention(qb, kb, vb, kv_lens[b], windows, scale)
        assert np.max(np.abs(o - ob)) < 1e-12
        assert np.max(np.abs(lse - lb)) < 1e-12


def test_attend_batch_row_subsets_follow_the_requested_order():
    q, k, v, cu_q, cu_kv, kv_lens, q_lens = _varlen_batch(8)
    windows, scale = (0, 4), 0.6
    rows = [np.array([12, 0, 7, 3, 11]), np.array([3, 1]), np.array([], dtype=np.int64), np.array([0])]
    outs = A.attend_batch(q, k, v, cu_q, cu_kv, windows, scale, rows_per_seq=rows)
    for b, (o, lse) in enumerate(outs):
        assert o.shape[0] == len(rows[b])
        if len(rows[b]) == 0:
            continue
        qb = A.bf16_bits_to_f64(q[cu_q[b]:cu_q[b + 1]])
        kb = A.bf16_bits_to_f64(k[cu_kv[b]:cu_kv[b + 1]])
        vb = A.bf16_bits_to_f64(v[cu_kv[b]:cu_kv[b + 1]])
        ob, lb = brute_attention(qb, kb, vb, kv_lens[b], windows, scale)
        assert np.max(np.abs(o - ob[rows[b]])) < 1e-12
        assert np.max(np.abs(lse - lb[rows[b]])) < 1e-12


@pytest.mark.parametrize("row_block", [1, 3, 256])
def test_row_subset_equals_the_same_rows_of_the_full_call(row_block):
    """Scattered, unsorted rows with repeats, across small row blocks: the
    subset path gives the full call's rows (up to the summation order of the
    columns it multiplies) in the order asked for."""
    rng = np.random.default_rng(31)
    kv_len, q_len, hq, hkv, d = 150, 90, 4, 2, 8
    q = A.bf16_bits_to_f64(_bits(rng, (q_len, hq, d), 2.0))
    k = A.bf16_bits_to_f64(_bits(rng, (kv_len, hkv, d)))
    v = A.bf16_bits_to_f64(_bits(rng, (kv_len, hkv, d)))
    windows, scale = (0, 17), 0.3
    o_full, l_full = A.attend_sequence(q, k, v, windows, scale)
    rows = np.array([89, 0, 45, 44, 1, 88, 60, 60, 17, 2, 70])
    o, lse = A.attend_sequence(q, k, v, windows, scale, rows=rows, row_block=row_block)
    assert o.shape == (len(rows), hq, d)
    assert np.max(np.abs(o - o_full[rows])) < 1e-13
    assert np.max(np.abs(lse - l_full[rows])) < 1e-13
    # and against brute force, independently of the blocked path
    ob, lb = brute_attention(q, k, v, kv_len, windows, scale)
    assert np.max(np.abs(o - ob[rows])) < 1e-12
    assert np.max(np.abs(lse - lb[rows])) < 1e-12


def test_relocated_batch_uses_each_sequences_own_offsets():
    q, k, v, cu_q, cu_kv, kv_lens, q_lens = _varlen_batch(9)
    windows, scale, theta = (0, 5), 0.5, 500.0
    deltas = [(0, 7), (3, -11), (100, 2), (0, 40)]  # distinct per sequence and per KV head
    rows = [np.array([12, 5, 0]), None, None, None]
    outs = RP.attend_batch_relocated(q, k, v, cu_q, cu_kv, windows, scale, deltas, theta, style=0,
                                     rope_dims=0, rows_per_seq=[r if r is not None else np.arange(n)
                                                                for r, n in zip(rows, q_lens)])
    hq, hkv = q.shape[1], k.shape[1]
    grp = hq // hkv
    for b, (o, lse) in enumerate(outs):
        if q_lens[b] == 0:
            assert o.shape[0] == 0
            continue
        qb = A.bf16_bits_to_f64(q[cu_q[b]:cu_q[b + 1]])
        kb = A.bf16_bits_to_f64(k[cu_kv[b]:cu_kv[b + 1]])
        vb = A.bf16_bits_to_f64(v[cu_kv[b]:cu_kv[b + 1]])
        o1, l1 = RP.attend_sequence_relocated(qb, kb, vb, windows, scale, deltas[b], theta)
        qr = qb.copy()
        for g in range(hkv):
            qr[:, g * grp:(g + 1) * grp] = RP.relocate_queries(qb[:, g * grp:(g + 1) * grp], deltas[b][g], theta)
        ob, lb = brute_attention(qr, kb, vb, kv_lens[b], windows, scale)
        sel = rows[b] if rows[b] is not None else np.arange(q_lens[b])
        assert np.max(np.abs(o - o1[sel])) < 1e-13
        assert np.max(np.abs(o - ob[sel])) < 1e-12
        assert np.max(np.abs(lse - lb[sel])) < 1e-12
        # another sequence's offsets would give a different result
        if any(deltas[b]):
            other = deltas[(b + 1) % len(deltas)]
            o2, _ = RP.attend_sequence_relocated(qb, kb, vb, windows, scale, other, theta)
            assert np.max(np.abs(o2[sel] - o)) > 1e-3


def test_paged_store_is_not_the_identity_and_the_table_matters():
    """The placement pin is not vacuous: the pool holds pages out of logical
    order, gathering through the right table returns the rows exactly, and a
    wrong table (two entries swapped) changes both the rows and the result."""
    rng = np.random.default_rng(5)
    kv_len, d, page = 70, 8, 16
    q = A.bf16_bits_to_f64(_bits(rng, (kv_len, 2, d)))
    k = A.bf16_bits_to_f64(_bits(rng, (kv_len, 2, d)))
    v = A.bf16_bits_to_f64(_bits(rng, (kv_len, 2, d)))
    pool_k, table = A.paged_store(k, page, 3)
    pool_v, table_v = A.paged_store(v, page, 3)
    np.testing.assert_array_equal(table, table_v)
    flat = pool_k.reshape((-1,) + k.shape[1:])[:kv_len]
    assert not np.array_equal(flat, k)                       # physical order differs
    np.testing.assert_array_equal(A.paged_gather(pool_k, table, kv_len), k)
    wrong = table.copy()
    wrong[[0, 2]] = wrong[[2, 0]]
    kw = A.paged_gather(pool_k, wrong, kv_len)
    vw = A.paged_gather(pool_v, wrong, kv_len)
    assert not np.array_equal(kw, k)
    o0, l0 = A.attend_sequence(q, k, v, (0, 9), 0.3)
    ow, lw = A.attend_sequence(q, kw, vw, (0, 9), 0.3)
    assert np.max(np.abs(ow - o0)) > 1e-3 and np.max(np.abs(lw - l0)) > 1e-3
    kr, t2 = A.paged_round_trip(k, page, 3)
    np.testing.assert_array_equal(kr, k)
    np.testing.assert_array_equal(t2, table)
