"""Pins of the attention-mass token score oracle.

* a pure-Python brute force with math.exp over explicit loops;
* the mass over all keys is exactly (query rows) x (query heads): every
  probability row sums to 1;
* Q = 0 (uniform attention over the visible keys) has a harmonic-sum
  closed form per key;
* a planted key that every row favours gets the top score;
* top-k against numpy's stable argsort on distinct scores, and ties going
  to the lower index.
"""

import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import router as RT


def brute_scores(q, k, windows, scale):
    q_len, hq, d = q.shape
    kv_len, hkv, _ = k.shape
    g_size = hq // hkv
    mass = [0.0] * kv_len
    for t in range(q_len):
        p = kv_len - q_len + t
        for h in range(hq):
            g = h // g_size
            vis = [j for j in range(kv_len) if A.is_visible(p, j, windows[g])]
            s = {j: scale * sum(q[t, h, c] * k[j, g, c] for c in range(d)) for j in vis}
            mx = max(s.values())
            z = sum(math.exp(s[j] - mx) for j in vis)
            for j in vis:
                mass[j] += math.exp(s[j] - mx) / z
    return np.array(mass)


@pytest.mark.parametrize("kv,q,hq,hkv,windows", [(9, 9, 2, 1, (0,)), (12, 5, 4, 2, (0, 3)), (20, 7, 3, 3, (1, 0, 6))])
def test_scores_match_brute_force(kv, q, hq, hkv, windows):
    rng = np.random.default_rng(kv + q)
    qq = rng.standard_normal((q, hq, 4))
    kk = rng.standard_normal((kv, hkv, 4))
    full = RT.token_scores(qq, kk, windows, 0.7, all_keys=True)
    np.testing.assert_allclose(full, brute_scores(qq, kk, windows, 0.7), atol=1e-12)
    np.testing.assert_array_equal(RT.token_scores(qq, kk, windows, 0.7), full[kv - q:])


def test_total_mass_is_rows_times_heads():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((40, 8, 16)) * 3
    k = rng.standard_normal((100, 2, 16))
    full = RT.token_scores(q, k, (0, 17), 0.25, all_keys=True)
    assert abs(full.sum() - 40 * 8) < 1e-9
    assert np.all(full >= 0)


def test_uniform_attention_closed_form():
    """Q = 0: a row at position p spreads mass 1/n(p) over its n(p) visible
    keys, so key j gets G * sum over rows p that see j of 1/n(p)."""
    kv, ql, hq, hkv, d = 50, 30, 6, 2, 8
    windows = (0, 7)
    k = np.random.default_rng(2).standard_normal((kv, hkv, d))
    got = RT.token_scores(np.zeros((ql, hq, d)), k, windows, 1.0, all_keys=True)
    want = np.zeros(kv)
    for w in windows:
        for p in range(kv - ql, kv):
            lo = 0 if w == 0 else max(0, p - w + 1)
            want[lo:p + 1] += (hq // hkv) / (p + 1 - lo)
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_planted_key_gets_the_top_score():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((64, 4, 32))
    k = rng.standard_normal((64, 1, 32)) * 0.1
    k[5, 0] = q[:, :, :].mean(axis=(0, 1)) * 20  # aligned with every query
    s = RT.token_scores(q, k, (0,), 1 / math.sqrt(32))
    assert int(np.argmax(s)) == 5
    assert 5 in RT.top_k(s, 1)


def test_top_k_against_argsort_and_ties():
    rng = np.random.default_rng(4)
    s = rng.standard_normal(300)
    for k in (0, 1, 17, 300):
        want = np.sort(np.argsort(-s, kind="stable")[:k])
        np.testing.assert_array_equal(RT.top_k(s, k), want)
    tied = np.array([1.0, 3.0, 2.0, 3.0, 3.0, 0.5])
    np.testing.assert_array_equal(RT.top_k(tied, 2), [1, 3])
    np.testing.assert_array_equal(RT.top_k(tied, 4), [1, 2, 3, 4])
