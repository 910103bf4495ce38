"""Pins of the head-decomposition merge oracle.

* the merge of partial attentions over two disjoint key sets equals a
  directly written softmax over their union;
* empty parts, symmetry, associativity and no overflow at extreme lse;
* selected rows are returned bit for bit;
* end to end: offline document-only outputs for Local heads, LSE-merged
  with a partial over the keys before the document on the window's
  boundary rows, and online recomputation for Global heads and protected
  rows, reproduce the attention of the whole request exactly.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import merge as M


def direct_softmax(q, k, v, scale):
    """softmax(scale q k^T) v and its lse, written out (q [D], k/v [n][D])."""
    s = scale * (k @ q)
    if len(s) == 0:
        return np.zeros(v.shape[1]), -np.inf
    mx = s.max()
    e = np.exp(s - mx)
    return (e @ v) / e.sum(), mx + np.log(e.sum())


def test_merge_of_disjoint_parts_is_the_union():
    rng = np.random.default_rng(0)
    d = 16
    for n1, n2 in ((5, 7), (1, 30), (40, 1), (0, 9)):
        q = rng.standard_normal(d)
        k = rng.standard_normal((n1 + n2, d))
        v = rng.standard_normal((n1 + n2, d))
        perm = rng.permutation(n1 + n2)  # the two sets need not be contiguous
        s1, s2 = perm[:n1], perm[n1:]
        o1, l1 = direct_softmax(q, k[s1], v[s1], 0.3)
        o2, l2 = direct_softmax(q, k[s2], v[s2], 0.3)
        ou, lu = direct_softmax(q, k, v, 0.3)
        om, lm = M.merge_pair(o1, l1, o2, l2)
        np.testing.assert_allclose(om, ou, atol=1e-13)
        np.testing.assert_allclose(lm, lu, atol=1e-13)


def test_empty_parts_symmetry_and_associativity():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((3, 8))
    lse = rng.standard_normal(3) * 5
    z_o, z_l = np.full((3, 8), 7.0), np.full(3, -np.inf)  # an empty part's o is ignored
    mo, ml = M.merge_pair(o, lse, z_o, z_l)
    np.testing.assert_array_equal(ml, lse)
    np.testing.assert_allclose(mo, o, atol=1e-15)
    eo, el = M.merge_pair(z_o, z_l, z_o, z_l)
    assert np.all(eo == 0) and np.all(np.isneginf(el))
    o2, l2 = rng.standard_normal((3, 8)), rng.standard_normal(3)
    o3, l3 = rng.standard_normal((3, 8)), rng.standard_normal(3)
    np.testing.assert_allclose(M.merge_pair(o, lse, o2, l2)[0], M.merge_pair(o2, l2, o, lse)[0], atol=1e-15)
    left = M.merge_pair(*M.merge_pair(o, lse, o2, l2), o3, l3)
    right = M.merge_pair(o, lse, *M.merge_pair(o2, l2, o3, l3))
    np.testing.assert_allclose(left[0], right[0], atol=1e-14)
    np.testing.assert_allclose(left[1], right[1], atol=1e-14)


def test_extreme_lse_does_not_overflow():
    o_a, o_b = np.ones((1, 4)), -np.ones((1, 4))
    o, l = M.merge_pair(o_a, np.array([1000.0]), o_b, np.array([-1000.0]))
    np.testing.assert_allclose(o, o_a, atol=1e-300)
    assert l[0] == 1000.0
    o, l = M.merge_pair(o_a, np.array([700.0]), o_b, np.array([700.0]))
    np.testing.assert_allclose(o, 0.0, atol=1e-15)
    np.testing.assert_allclose(l, 700.0 + np.log(2.0), rtol=1e-15)


def test_selected_rows_are_returned_bit_for_bit():
    rng = np.random.default_rng(2)
    o_a, o_b = rng.standard_normal((6, 3, 8)), rng.standard_normal((6, 3, 8))
    l_a, l_b = rng.standard_normal((6, 3)), rng.standard_normal((6, 3))
    mode = rng.integers(0, 3, size=(6, 3))
    o, l = M.head_decomposition_merge(o_a, l_a, o_b, l_b, mode)
    np.testing.assert_array_equal(o[mode == M.TAKE_A], o_a[mode == M.TAKE_A])
    np.testing.assert_array_equal(l[mode == M.TAKE_B], l_b[mode == M.TAKE_B])
    mo, ml = M.merge_pair(o_a, l_a, o_b, l_b)
    np.testing.assert_array_equal(o[mode == M.MERGE], mo[mode == M.MERGE])
    with pytest.raises(ValueError):
        M.head_decomposition_merge(o_a, l_a, o_b, l_b, np.full((6, 3), 3))


@pytest.mark.parametrize("a,n,window", [(40, 70, 16), (64, 64, 1), (10, 90, 100)])
def test_decomposition_reproduces_full_recomputation(a, n, window):
    """A request = a prefix of a tokens + a document of n tokens.  Heads of
    KV group 0 are global, those of group 1 local with the given window."""
    rng = np.random.default_rng(a + n + window)
    hq, hkv, d, scale = 4, 2, 16, 0.25
    windows = (0, window)
    q = rng.standard_normal((n, hq, d))          # the document's rows
    k = rng.standard_normal((a + n, hkv, d))
    v = rng.standard_normal((a + n, hkv, d))
    full_o, full_l = A.attend_sequence(q, k, v, windows, scale)        # live request
    off_o, off_l = A.attend_sequence(q, k[a:], v[a:], windows, scale)  # document alone, offline
    # online partial over the prefix keys only, for every (row, head)
    pre_o, pre_l = np.zeros((n, hq, d)), np.full((n, hq), -np.inf)
    for t in range(n):
        p = a + t
        for h in range(hq):
            g = h // (hq // hkv)
            lo = 0 if windows[g] == 0 else max(0, p - windows[g] + 1)
            keys = np.arange(lo, min(a, p + 1))
            pre_o[t, h], pre_l[t, h] = direct_softmax(q[t, h], k[keys, g], v[keys, g], scale)
    protected = np.zeros(n, bool)
    protected[::7] = True           # e.g. dirty rows
    protected[-5:] = True           # a tail
    mode = np.full((n, hq), M.TAKE_A)
    local = np.array([windows[h // (hq // hkv)] > 0 for h in range(hq)])
    boundary = (np.arange(n) < window - 1)[:, None] & local[None, :]   # local rows that also see prefix keys
    mode[boundary] = M.MERGE
    mode[:, ~local] = M.TAKE_B
    mode[protected, :] = M.TAKE_B
    # online path: full recomputation where selected, the prefix partial where merged
    on_o = np.where((mode == M.TAKE_B)[..., None], full_o, pre_o)
    on_l = np.where(mode == M.TAKE_B, full_l, pre_l)
    o, l = M.head_decomposition_merge(off_o, off_l, on_o, on_l, mode)
    np.testing.assert_allclose(o, full_o, atol=1e-12)
    np.testing.assert_allclose(l, full_l, atol=1e-12)
    # the offline output alone is wrong exactly where a local row sees prefix keys
    if a > 0 and window > 1:
        assert np.max(np.abs(off_l[boundary] - full_l[boundary])) > 1e-6
