"""Pins of the fp64 oracle against things other than itself.

Each check is chosen so that a plausible mistake in the oracle (a window off
by one, a wrong query offset, a swapped operand, a wrong GQA mapping, a base-2
log-sum-exp, a dropped normalisation) fails at least one of them:

* brute force: a separately written pure-Python loop on tiny inputs;
* a library routine: torch scaled_dot_product_attention in float64 on CPU
  with an explicit boolean mask (and is_causal for global heads);
* closed forms: zero queries give the mean of the visible values and
  lse = ln |visible|; W = 1 gives v_p; values that encode the key position
  give the exact mean visible position;
* invariants: W >= kv_len equals global, page placement does not matter,
  probabilities sum to one and vanish off the visible set, GQA equals MHA
  with repeated KV, merging split parts equals the whole, and the mask count
  equals the closed-form visible-pair ledger.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from long_context_serving_amd import workloads as wl
from oracle import attention as A
from oracle import ledger as LG
from oracle import segments as SG

from brute import brute_attention as _brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_bf16(rng, shape, scale=1.0):
    return wl.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


@pytest.mark.parametrize("case", [
    # kv_len, q_len, hq, hkv, d, windows
    (9, 9, 2, 2, 4, (0, 3)),
    (12, 5, 4, 2, 3, (1, 4)),        # chunked queries, GQA 2
    (7, 1, 3, 1, 5, (2,)),           # decode-like, one KV head
    (10, 10, 4, 4, 2, (0, 1, 10, 25)),
])
def test_oracle_matches_brute_force(case):
    kv_len, q_len, hq, hkv, d, windows = case
    rng = np.random.default_rng(hash(case) % 2**32)
    q = A.bf16_bits_to_f64(_rand_bf16(rng, (q_len, hq, d)))
    k = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, hkv, d)))
    v = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, hkv, d)))
    scale = 0.7
    o, lse = A.attend_sequence(q, k, v, windows, scale, row_block=3)
    ob, lb = _brute(q, k, v, kv_len, windows, scale)
    assert np.max(np.abs(o - ob)) < 1e-12
    assert np.max(np.abs(lse - lb)) < 1e-12


@pytest.mark.parametrize("kv_len,q_len,windows", [
    (64, 64, (0, 16)), (80, 24, (0, 9)), (33, 33, (5, 100)), (50, 1, (0, 7))])
def test_oracle_matches_torch_sdpa_fp64(kv_len, q_len, windows):
    rng = np.random.default_rng(kv_len * 131 + q_len)
    hq, hkv, d = 4, 2, 16
    q = A.bf16_bits_to_f64(_rand_bf16(rng, (q_len, hq, d)))
    k = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, hkv, d)))
    v = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, hkv, d)))
    scale = 1.0 / math.sqrt(d)
    o, lse = A.attend_sequence(q, k, v, windows, scale)
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [hq, q, d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    pos = torch.arange(kv_len - q_len, kv_len)[:, None]
    j = torch.arange(kv_len)[None, :]
    for h in range(hq):
        w = windows[h // (hq // hkv)]
        mask = j <= pos
        if w:
            mask = mask & (j > pos - w)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[h:h + 1], kt[h:h + 1], vt[h:h + 1], attn_mask=mask, scale=scale)
        assert torch.max(torch.abs(ref[0] - torch.from_numpy(o[:, h, :]))).item() < 1e-12
        s = scale * (qt[h] @ kt[h].T)
        ref_lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
        assert torch.max(torch.abs(ref_lse - torch.from_numpy(lse[:, h]))).item() < 1e-12
        if w == 0 and q_len == kv_len:
            ref_c = torch.nn.functional.scaled_dot_product_attention(
                qt[h:h + 1], kt[h:h + 1], vt[h:h + 1], is_causal=True, scale=scale)
            assert torch.max(torch.abs(ref_c[0] - torch.from_numpy(o[:, h, :]))).item() < 1e-12


@pytest.mark.parametrize("window", [0, 1, 5, 16, 40])
def test_zero_query_gives_mean_of_visible_values(window):
    kv_len, q_len, d = 40, 13, 8
    rng = np.random.default_rng(window + 3)
    q = np.zeros((q_len, 1, d))
    k = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, 1, d)))
    v = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, 1, d)))
    o, lse = A.attend_sequence(q, k, v, (window,), 0.3)
    for t in range(q_len):
        p = kv_len - q_len + t
        lo = 0 if window == 0 else max(0, p - window + 1)
        n = p - lo + 1
        assert n == (p + 1 if window == 0 else min(p + 1, window))
        np.testing.assert_allclose(o[t, 0], v[lo:p + 1, 0].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[t, 0] - math.log(n)) < 1e-13


def test_window_one_returns_own_value_and_score():
    kv_len, q_len, d = 30, 30, 16
    rng = np.random.default_rng(7)
    q = A.bf16_bits_to_f64(_rand_bf16(rng, (q_len, 2, d)))
    k = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, 1, d)))
    v = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, 1, d)))
    scale = 0.25
    o, lse = A.attend_sequence(q, k, v, (1,), scale)
    for t in range(q_len):
        for h in range(2):
            np.testing.assert_array_equal(o[t, h], v[t, 0])
            assert abs(lse[t, h] - scale * float(q[t, h] @ k[t, 0])) < 1e-13


@pytest.mark.parametrize("kv_len,q_len,window", [(700, 700, 64), (700, 96, 130), (257, 40, 0), (300, 300, 1000)])
def test_position_encoding_values_give_mean_visible_position(kv_len, q_len, window):
    """v_j[0] = j mod 16, v_j[1] = j // 16 (exact in bf16); zero queries
    average them uniformly over the visible set, so 16*o[1] + o[0] is the
    mean visible key position, known in closed form: (lo + p) / 2."""
    d = 4
    q = np.zeros((q_len, 1, d))
    k = np.zeros((kv_len, 1, d))
    v = np.zeros((kv_len, 1, d))
    j = np.arange(kv_len)
    v[:, 0, 0] = j % 16
    v[:, 0, 1] = j // 16
    o, _ = A.attend_sequence(q, k, v, (window,), 1.0)
    for t in range(q_len):
        p = kv_len - q_len + t
        lo = 0 if window == 0 else max(0, p - window + 1)
        assert abs(16 * o[t, 0, 1] + o[t, 0, 0] - (lo + p) / 2) < 1e-9


def test_wide_local_window_equals_global_bitwise():
    kv_len, q_len, d = 48, 20, 8
    rng = np.random.default_rng(11)
    q = A.bf16_bits_to_f64(_rand_bf16(rng, (q_len, 4, d)))
    k = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, 2, d)))
    v = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, 2, d)))
    og, lg = A.attend_sequence(q, k, v, (0, 0), 0.5)
    for w in (kv_len, kv_len + 1, 10 * kv_len):
        ol, ll = A.attend_sequence(q, k, v, (w, w), 0.5)
        np.testing.assert_array_equal(og, ol)
        np.testing.assert_array_equal(lg, ll)


def test_page_placement_does_not_matter():
    kv_len, d = 70, 8
    rng = np.random.default_rng(5)
    q = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, 2, d)))
    k = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, 2, d)))
    v = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, 2, d)))
    o0, l0 = A.attend_sequence(q, k, v, (0, 9), 0.3)
    for seed in (1, 2, 3):
        kp, perm = A.paged_round_trip(k, 16, seed)
        vp, _ = A.paged_round_trip(v, 16, seed)
        assert not np.array_equal(perm, np.arange(len(perm)))
        o1, l1 = A.attend_sequence(q, kp, vp, (0, 9), 0.3)
        np.testing.assert_array_equal(o0, o1)
        np.testing.assert_array_equal(l0, l1)


@pytest.mark.parametrize("window", [0, 1, 6])
def test_probabilities_sum_to_one_and_vanish_off_visible_set(window):
    """With V = identity the output row is the probability row itself."""
    kv_len, q_len, d = 25, 25, 6
    rng = np.random.default_rng(window)
    q = A.bf16_bits_to_f64(_rand_bf16(rng, (q_len, d), 2.0))
    k = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, d)))
    pos = A.query_positions(kv_len, q_len)
    mask = A.visibility_mask(pos, kv_len, window)
    probs, _ = A.masked_softmax_attention(q, k, np.eye(kv_len), mask, 0.9)
    assert np.all(np.abs(probs.sum(axis=1) - 1.0) <= 1e-12)
    assert np.all(probs[~mask] == 0.0)
    assert np.all(probs[mask] > 0.0)


def test_gqa_equals_mha_with_repeated_kv():
    kv_len, q_len, d = 33, 17, 8
    rng = np.random.default_rng(21)
    q = A.bf16_bits_to_f64(_rand_bf16(rng, (q_len, 8, d)))
    k = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, 2, d)))
    v = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, 2, d)))
    o, l = A.attend_sequence(q, k, v, (0, 5), 0.4)
    k8 = np.repeat(k, 4, axis=1)
    v8 = np.repeat(v, 4, axis=1)
    o8, l8 = A.attend_sequence(q, k8, v8, (0,) * 4 + (5,) * 4, 0.4)
    np.testing.assert_array_equal(o, o8)
    np.testing.assert_array_equal(l, l8)


def test_merging_split_parts_equals_whole():
    kv_len, q_len, d = 90, 30, 8
    rng = np.random.default_rng(9)
    q = A.bf16_bits_to_f64(_rand_bf16(rng, (q_len, d), 3.0))
    k = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, d)))
    v = A.bf16_bits_to_f64(_rand_bf16(rng, (kv_len, d)))
    pos = A.query_positions(kv_len, q_len)
    mask = A.visibility_mask(pos, kv_len, 40)
    o_full, l_full = A.masked_softmax_attention(q, k, v, mask, 0.35)
    cuts = [0, 7, 31, 55, 56, 90]            # includes an empty part for some rows
    o_parts, l_parts = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        sub = np.zeros_like(mask)
        sub[:, a:b] = mask[:, a:b]
        rows = sub.any(axis=1)
        op = np.zeros((q_len, d))
        lp = np.full(q_len, -np.inf)
        if rows.any():
            op[rows], lp[rows] = A.masked_softmax_attention(q[rows], k, v, sub[rows], 0.35)
        o_parts.append(op)
        l_parts.append(lp)
    assert np.isneginf(np.array(l_parts)).any()
    o_m, l_m = A.merge_partials(np.array(o_parts), np.array(l_parts))
    assert np.max(np.abs(o_m - o_full)) < 1e-12
    assert np.max(np.abs(l_m - l_full)) < 1e-12


@pytest.mark.parametrize("kv_len,q_len,window", [
    (512, 512, 64), (512, 512, 0), (100, 30, 7), (100, 30, 200), (64, 1, 64), (65, 1, 64),
    (1, 1, 1), (1000, 1000, 1000), (1000, 999, 999), (1000, 0, 5)])
def test_mask_count_equals_ledger(kv_len, q_len, window):
    pos = A.query_positions(kv_len, q_len)
    assert int(A.visibility_mask(pos, kv_len, window).sum()) == LG.visible_pairs(kv_len, q_len, window)
    assert sum(LG.visible_count(int(p), window) for p in pos) == LG.visible_pairs(kv_len, q_len, window)


def test_ledger_flops_of_named_workloads():
    # visible-pair sums checked term by term against the per-position count
    w = wl.MISTRAL7B_PREFILL
    pairs = sum(w.group * sum(min(p + 1, x) if x else p + 1 for p in range(8192)) for x in w.windows)
    assert LG.prefill_visible_flops(w.kv_lens, w.q_lens, w.windows, w.num_q_heads, w.head_dim) == 4 * 128 * pairs
    assert pairs == 354_449_408
    d = wl.DECODE_32K
    by = LG.decode_visible_bytes(d.kv_lens, d.windows, d.num_q_heads, d.head_dim)
    assert by["kv"] == 31 * (32768 + 7 * 4096) * 128 * 2 * 2


def test_head_row_ceilings_printed_on_pages():
    with open(os.path.join(GOLDEN, "head_row_ceilings.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = 100 * LG.head_row_ceiling(c["reusable_layers"], c["total_layers"],
                                        c["local_heads"], c["total_heads"])
        assert round(got, 2) == c["ceiling_percent"]


def _brute_needed_min(kv_len, n_query, window, horizon=64):
    """Smallest key any query at a pending or future position can see,
    by enumeration of positions and keys."""
    p_q = kv_len - n_query
    best = None
    for p in range(p_q, kv_len + horizon):
        for j in range(0, p + 1):
            if window == 0 or j > p - window:
                best = j if best is None else min(best, j)
    return best


@pytest.mark.parametrize("kv_len,n_query,window,page", [
    (40, 40, 8, 4), (40, 0, 8, 4), (40, 3, 8, 16), (100, 1, 37, 16), (100, 0, 0, 16),
    (17, 5, 1, 4), (33, 0, 33, 8), (33, 0, 34, 8), (5, 5, 100, 16)])
def test_segment_start_matches_enumeration(kv_len, n_query, window, page):
    lo = _brute_needed_min(kv_len, n_query, window)
    first = SG.segment_first_token(kv_len, n_query, window, page)
    assert first == page * (lo // page)
    assert first <= lo < first + page
    n_pages = SG.segment_pages(kv_len, first, page)
    assert first + n_pages * page >= kv_len > first + (n_pages - 1) * page


def test_segment_never_moves_back_and_matches_named_workload():
    # a decode-at-32K sequence: fill 32767 tokens with no queries, then one decode token
    kv, first, pages = SG.segment_after_appends([(32767, 0), (1, 1)], 4096, 64)
    assert (kv, first, pages) == (32768, 28672, 64)
    kv, first, pages = SG.segment_after_appends([(32767, 0), (1, 1)], 0, 64)
    assert (first, pages) == (0, 512)
    # one-shot prefill keeps everything, the next decode token trims
    assert SG.segment_after_appends([(8192, 8192)], 1024, 64)[2] == 128
    assert SG.segment_after_appends([(8192, 8192), (1, 1)], 1024, 64)[1:] == (7168, 17)


def test_bf16_decoding_is_exact():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x3E80], dtype=np.uint16)
    vals = A.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[2] == 2.0 ** -133
    assert vals[3] == (2 - 2 ** -7) * 2.0 ** 127 and vals[4] == 0.0 and vals[5] == 0.25
