"""The seeded input generator: bf16 rounding and the named shapes."""

import numpy as np

from long_context_serving_amd import metrics as M
from long_context_serving_amd import workloads as wl


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is exactly half way between 1 and 1 + 2^-7: ties go to even (1.0)
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5, 3.0e-39], dtype=np.float32)
    b = wl.to_bf16_bits(x)
    assert b[0] == 0x3F80
    assert b[1] == 0x3F80                 # tie -> even mantissa
    assert b[2] == 0x3F82                 # tie -> even (odd 0x3F81 loses)
    assert b[3] == 0x3F81                 # above half way -> up
    assert b[4] == 0xC020
    # subnormal float32 rounds like any other value
    assert b[5] == (np.array([3.0e-39], dtype=np.float32).view(np.uint32)[0] + 0x7FFF
                    + ((np.array([3.0e-39], dtype=np.float32).view(np.uint32)[0] >> 16) & 1)) >> 16


def test_named_workload_shapes():
    assert wl.LLAMA70B_VARLEN_PREFILL.kv_lens == (29127, 12589, 8841, 23919)
    assert wl.DECODE_32K.fill_lens() == (32767,) * 31
    assert wl.CHUNKED_PREFILL_128K.fill_lens() == (122880,)
    assert wl.TINY_MHA.windows == (0, 64, 64, 64)
    assert wl.MISTRAL7B_PREFILL.all_global().windows == (0,) * 8


def test_inputs_are_seeded_and_shaped():
    w = wl.small_workload("t", (10, 3), (4, 3), 4, 2, 8, 16, (0, 3), seed=42)
    a = wl.make_inputs(w)
    b = wl.make_inputs(w)
    assert a.q.shape == (7, 4, 8) and a.k.shape == (13, 2, 8) and a.v.shape == (13, 2, 8)
    assert a.q.dtype == np.uint16
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.cu_q, [0, 4, 7])
    np.testing.assert_array_equal(a.cu_kv, [0, 10, 13])
    c = wl.make_inputs(w, seed=43)
    assert not np.array_equal(a.k, c.k)


def test_product_ledger_matches_oracle_closed_forms():
    from long_context_serving_amd import metrics as M
    from oracle import ledger as LG
    for w in wl.WORKLOADS.values():
        for windows in (w.windows, (0,) * w.num_kv_heads):
            if w.decode:
                assert M.decode_bytes(w, windows) == LG.decode_visible_bytes(
                    w.kv_lens, windows, w.num_q_heads, w.head_dim)
            else:
                assert M.prefill_flops(w, windows) == LG.prefill_visible_flops(
                    w.kv_lens, w.q_lens, windows, w.num_q_heads, w.head_dim)
    w = wl.MISTRAL7B_PREFILL
    assert M.prefill_flops(w) == 181_478_096_896
    rows = np.arange(0, 8192, 97)
    assert M.prefill_flops_rows(w, 0, rows) == 4 * 128 * 4 * sum(
        min(p + 1, x) if x else p + 1 for p in rows for x in w.windows)


def test_merge_modes_follow_the_recipe():
    mw = wl.MergeWorkload("m", 2000, 16, 4, 64, window=300, tail=256, query_rows=40, boundary_every=128,
                          dirty_frac=0.03, seed=3)
    mode = wl.merge_modes(mw)
    assert mode.shape == (2000, 16) and mode.dtype == np.uint8
    assert np.all(mode[:, :4] == wl.TAKE_B)            # KV head 0's query heads are global
    local = mode[:, 4:]
    assert np.all(local[::128] == wl.TAKE_B)
    assert np.all(local[-256:] == wl.TAKE_B)
    unprotected = np.all(local != wl.TAKE_B, axis=1)
    assert np.all(local[:299][unprotected[:299]] == wl.MERGE)
    assert np.all(local[299:][unprotected[299:]] == wl.TAKE_A)
    dirty = np.flatnonzero(~unprotected[:-256])
    dirty = dirty[dirty % 128 != 0]
    assert 0.01 < len(dirty) / 2000 < 0.05


def test_merge_bytes_against_per_pair_count():
    rng = np.random.default_rng(0)
    mode = rng.integers(0, 3, size=(50, 6)).astype(np.uint8)
    d = 64
    read = write = 0
    for m in mode.ravel():
        read += 1 + (d * 2 + 4) * (2 if m == 2 else 1)
        write += d * 2 + 4
    b = M.merge_bytes(mode, d)
    assert (b["read"], b["write"], b["total"]) == (read, write, read + write)
    assert b["take_a"] + b["take_b"] + b["merge"] == b["pairs"] == 300
