"""Pins of the RoPE relocation oracle.

* an independently written complex-number form of the rotation;
* inverse and composition identities;
* the relative-position property the relocation relies on;
* end to end: keys encoded at canonical positions (document at 0) with
  queries turned back by the document offset give the same attention as
  keys and queries encoded at their true positions (full recomputation).
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import rope as RP


def test_rotation_matches_complex_multiplication():
    rng = np.random.default_rng(0)
    d, theta = 16, 10000.0
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 7, 1000, 123457])
    z = x[:, : d // 2] + 1j * x[:, d // 2:]
    w = np.exp(1j * pos[:, None] * theta ** (-np.arange(d // 2) * 2.0 / d))
    zr = z * w
    ref = np.concatenate([zr.real, zr.imag], axis=1)
    np.testing.assert_allclose(RP.rope_rotate(x, pos, theta), ref, rtol=0, atol=1e-12)


def test_inverse_and_composition():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 128))
    for th in (10000.0, 500000.0):
        np.testing.assert_allclose(RP.rope_rotate(RP.rope_rotate(x, 977, th), -977, th), x, atol=1e-12)
        np.testing.assert_allclose(RP.rope_rotate(RP.rope_rotate(x, 300, th), 45, th),
                                   RP.rope_rotate(x, 345, th), atol=1e-11)
        np.testing.assert_array_equal(RP.rope_rotate(x, 0, th), x)


def test_scores_depend_only_on_position_difference():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for p, j, delta in ((500, 17, 300), (9000, 8999, 8000), (5, 5, 5)):
        s_true = RP.rope_rotate(q, p, 10000.0) @ RP.rope_rotate(k, j, 10000.0)
        s_shift = RP.rope_rotate(q, p - delta, 10000.0) @ RP.rope_rotate(k, j - delta, 10000.0)
        assert abs(s_true - s_shift) < 1e-10


@pytest.mark.parametrize("delta,window", [(0, 0), (37, 0), (1000, 16), (250, 0)])
def test_canonical_keys_with_relocated_queries_equal_recomputation(delta, window):
    """A document of n tokens sits at offset delta.  Its keys were encoded at
    canonical positions 0..n-1; queries arrive encoded at their absolute
    positions delta + t.  Relocating the queries by -delta reproduces the
    attention of keys encoded at their true positions."""
    rng = np.random.default_rng(delta + window)
    n, hq, hkv, d, theta = 40, 4, 2, 32, 10000.0
    raw_q = rng.standard_normal((n, hq, d))
    raw_k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    pos_true = delta + np.arange(n)
    q_abs = RP.rope_rotate(raw_q, pos_true[:, None], theta)
    k_true = RP.rope_rotate(raw_k, pos_true[:, None], theta)
    k_canon = RP.rope_rotate(raw_k, np.arange(n)[:, None], theta)
    windows = (0, window)
    ref_o, ref_l = A.attend_sequence(q_abs, k_true, v, windows, 0.2)
    got_o, got_l = RP.attend_sequence_relocated(q_abs, k_canon, v, windows, 0.2, (delta, delta), theta)
    np.testing.assert_allclose(got_o, ref_o, atol=1e-10)
    np.testing.assert_allclose(got_l, ref_l, atol=1e-10)
    if delta:
        # without the relocation the result is different
        bad_o, _ = A.attend_sequence(q_abs, k_canon, v, windows, 0.2)
        assert np.max(np.abs(bad_o - ref_o)) > 1e-3


def test_zero_delta_heads_are_untouched():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((10, 4, 16))
    k = rng.standard_normal((10, 2, 16))
    v = rng.standard_normal((10, 2, 16))
    o1, l1 = RP.attend_sequence_relocated(q, k, v, (0, 3), 0.3, (0, 0), 10000.0)
    o2, l2 = A.attend_sequence(q, k, v, (0, 3), 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
