"""Copy-on-write forks in the product allocator, driven through the C ABI in
a planning-only context (host logic only), checked operation by operation
against the token-level fork model of the oracle."""

import os

import numpy as np
import pytest

from long_context_serving_amd import segkv as S
from long_context_serving_amd.build import LIB_PATH
from oracle import fork as F


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(LIB_PATH):
        from long_context_serving_amd.build import build
        build()
    S.load_library()


def planning_ctx(windows, page, pages, seqs):
    return S.SegKV(num_layers=1, num_q_heads=len(windows), num_kv_heads=len(windows), head_dim=64,
                   page_size=page, max_seqs=seqs, num_pages=pages, head_window=list(windows), planning=True)


def compare(kv, model, windows, seqs):
    assert kv.num_pages - kv.free_pages() == model.pages_in_use()
    id_to_obj, obj_to_id = {}, {}
    for s in range(seqs):
        for g in range(len(windows)):
            ft, kl, ids = kv.page_table(0, s, g)
            mf, mk, pages = model.segment(s, g)
            assert (kl, len(ids)) == (mk, len(pages)), (s, g)
            if len(ids):
                assert ft == mf, (s, g)
            for pid, pg in zip(ids.tolist(), pages):
                assert id_to_obj.setdefault(pid, id(pg)) == id(pg), "one page id stands for two model pages"
                assert obj_to_id.setdefault(id(pg), pid) == pid, "one model page has two page ids"


@pytest.mark.parametrize("seed", range(8))
def test_random_appends_forks_and_releases_match_the_model(seed):
    rng = np.random.default_rng(seed)
    windows = (0, 20, 70)
    P, seqs = 16, 6
    kv = planning_ctx(windows, P, 100_000, seqs)
    model = F.ForkModel(windows, P)
    label = 0
    for _ in range(120):
        op = rng.random()
        s = int(rng.integers(0, seqs))
        if op < 0.55:
            n_new = int(rng.integers(0, 50))
            n_q = int(rng.integers(0, n_new + 1))
            kv.append_pages(0, [s], [n_new], [n_q])
            model.append(s, list(range(label, label + n_new)), n_q)
            label += n_new
        elif op < 0.85:
            d = int(rng.integers(0, seqs))
            if d == s:
                with pytest.raises(S.SegKVError):
                    kv.fork(s, d)
            elif model.kv_len(d) == 0:
                kv.fork(s, d)
                model.fork(s, d)
            else:
                with pytest.raises(S.SegKVError) as e:
                    kv.fork(s, d)
                assert e.value.code == S.SEGKV_E_STATE
        else:
            kv.release(s)
            model.release(s)
        compare(kv, model, windows, seqs)


def test_batched_append_of_forks_matches_the_model():
    windows, P = (0, 40), 16
    kv = planning_ctx(windows, P, 10_000, 4)
    model = F.ForkModel(windows, P)
    kv.append_pages(0, [0], [75], [0])
    model.append(0, list(range(75)), 0)
    for d in (1, 2, 3):
        kv.fork(0, d)
        model.fork(0, d)
    compare(kv, model, windows, 4)
    kv.append_pages(0, [0, 1, 2, 3], [1, 30, 0, 5], [1, 2, 0, 5])
    for s, (n, q) in enumerate(((1, 1), (30, 2), (0, 0), (5, 5))):
        model.append(s, [f"{s}-{i}" for i in range(n)], q)
    compare(kv, model, windows, 4)


def test_pages_freed_by_every_holder_in_one_call_are_reusable():
    """A page shared by a sequence and its fork, dropped by both in one
    batched append, counts as free for that append."""
    kv = planning_ctx((16,), 16, 2, 2)
    kv.append_pages(0, [0], [16], [16])
    kv.fork(0, 1)
    assert kv.free_pages() == 1
    kv.append_pages(0, [0, 1], [16, 16], [1, 1])  # both windows move past the shared page
    assert kv.free_pages() == 0
    assert len(kv.page_table(0, 0, 0)[2]) == 1 and len(kv.page_table(0, 1, 0)[2]) == 1


def test_copy_on_write_needs_a_page_and_fails_whole():
    kv = planning_ctx((0,), 16, 2, 2)
    kv.append_pages(0, [0], [20], [0])   # 2 pages, the second holds 4 tokens
    kv.fork(0, 1)
    before = [kv.page_table(0, s, 0) for s in (0, 1)]
    with pytest.raises(S.SegKVError) as e:
        kv.append_pages(0, [1], [1], [1])  # needs a private copy of the shared tail
    assert e.value.code == S.SEGKV_E_NOMEM
    after = [kv.page_table(0, s, 0) for s in (0, 1)]
    assert all(b[:2] == a[:2] and np.array_equal(b[2], a[2]) for b, a in zip(before, after))
    kv.release(0)                          # the fork is now the only holder: no copy needed
    kv.append_pages(0, [1], [1], [1])
    assert kv.free_pages() == 0


def test_fork_argument_errors():
    kv = planning_ctx((0,), 16, 10, 2)
    for a, b in ((0, 2), (-1, 0)):
        with pytest.raises(S.SegKVError) as e:
            kv.fork(a, b)
        assert e.value.code == S.SEGKV_E_RANGE
