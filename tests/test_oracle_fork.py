"""Pins of the copy-on-write fork model.

* without forks it is the segment oracle (start, length, page count);
* every segment stores exactly its own sequence's tokens after any mix of
  appends, forks and releases (a shared page written without a copy breaks
  this);
* closed-form page counts for k forks of one parent that each append m
  tokens;
* a fork alone uses no page; releasing the forks gives the pages back.
"""

import numpy as np
import pytest

from oracle import fork as F
from oracle import segments as SG


def test_without_forks_it_is_the_segment_oracle():
    rng = np.random.default_rng(0)
    for _ in range(20):
        windows = (0, int(rng.integers(1, 200)), int(rng.integers(1, 40)))
        P = int(rng.choice([4, 16]))
        m = F.ForkModel(windows, P)
        appends = []
        for _ in range(int(rng.integers(1, 6))):
            n_new = int(rng.integers(0, 90))
            n_q = int(rng.integers(0, n_new + 1))
            appends.append((n_new, n_q))
            m.append("s", list(range(m.kv_len("s"), m.kv_len("s") + n_new)), n_q)
        for g, w in enumerate(windows):
            first, n, pages = m.segment("s", g)
            assert (n, first, len(pages)) == SG.segment_after_appends(appends, w, P)


def random_ops(seed, windows, P, n_ops=60, seqs=5):
    rng = np.random.default_rng(seed)
    m = F.ForkModel(windows, P)
    label = [0]
    for _ in range(n_ops):
        op = rng.random()
        s = int(rng.integers(0, seqs))
        if op < 0.55:
            n_new = int(rng.integers(0, 40))
            labels = list(range(label[0], label[0] + n_new))
            label[0] += n_new
            m.append(s, labels, int(rng.integers(0, n_new + 1)))
        elif op < 0.85:
            d = int(rng.integers(0, seqs))
            if d != s and m.kv_len(d) == 0:
                m.fork(s, d)
        else:
            m.release(s)
        yield m


@pytest.mark.parametrize("seed", range(6))
def test_every_segment_stores_its_own_history(seed):
    windows, P = (0, 7, 33), 8
    for m in random_ops(seed, windows, P):
        for (s, g) in list(m.segs):
            first, n, _ = m.segment(s, g)
            assert m.stored_labels(s, g) == m.history[s][first:n]


def test_a_model_without_the_copy_fails_the_history_check():
    """Plant the mistake: a model that writes shared pages in place.  After
    a fork, the child's append fills slots of the parent's tail page and the
    parent's next append overwrites them."""
    class NoCopy(F.ForkModel):
        def _refs(self, page):
            return 1

    for model, ok in ((F.ForkModel((0,), 16), True), (NoCopy((0,), 16), False)):
        model.append("p", list(range(10)), 0)
        model.fork("p", "c")
        model.append("c", [100, 101], 0)
        model.append("p", [200, 201], 0)
        good = all(model.stored_labels(x, 0) == model.history[x] for x in ("p", "c"))
        assert good == ok


@pytest.mark.parametrize("n,m_new,k,P", [(100, 5, 3, 16), (96, 40, 4, 16), (17, 1, 2, 4), (64, 0, 3, 16)])
def test_page_counts_of_k_forks(n, m_new, k, P):
    model = F.ForkModel((0,), P)
    model.append("p", list(range(n)), 0)
    base = -(-n // P)
    assert model.pages_in_use() == base
    for i in range(k):
        model.fork("p", i)
    assert model.pages_in_use() == base  # a fork alone shares everything
    for i in range(k):
        model.append(i, [f"{i}-{j}" for j in range(m_new)], 0)
    r = n % P
    per_child = -(-(r + m_new) // P) if m_new else 0
    assert model.pages_in_use() == base + k * per_child
    for i in range(k):
        model.release(i)
    assert model.pages_in_use() == base


def test_fork_needs_an_empty_target():
    m = F.ForkModel((0,), 4)
    m.append("a", [1, 2], 0)
    m.append("b", [3], 0)
    with pytest.raises(ValueError):
        m.fork("a", "b")
