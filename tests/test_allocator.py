"""Per-head segment page allocator, driven through the C ABI in a
planning-only context (host logic only, no GPU), checked against the
segment oracle and against pool invariants."""

import os

import numpy as np
import pytest

from long_context_serving_amd import segkv as S
from long_context_serving_amd.build import LIB_PATH
from oracle import segments as SG


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(LIB_PATH):
        from long_context_serving_amd.build import build
        build()
    S.load_library()


def ctx(windows, page=64, pages=100_000, seqs=4, layers=1, seed=0, hq=None):
    hkv = len(windows) // layers
    return S.SegKV(num_layers=layers, num_q_heads=hq or hkv, num_kv_heads=hkv, head_dim=128, page_size=page,
                   max_seqs=seqs, num_pages=pages, head_window=windows, page_order_seed=seed, planning=True)


def owned_pages(kv, layers, seqs, hkv):
    out = []
    for l in range(layers):
        for s in range(seqs):
            for g in range(hkv):
                out.extend(kv.page_table(l, s, g)[2].tolist())
    return out


def check_pool(kv, layers, seqs, hkv):
    owned = owned_pages(kv, layers, seqs, hkv)
    assert len(owned) == len(set(owned)), "a page is owned twice"
    assert len(owned) + kv.free_pages() == kv.num_pages
    assert all(0 <= p < kv.num_pages for p in owned)


def test_one_shot_prefill_then_decode_trims_local_heads():
    w = [0] + [1024] * 7
    kv = ctx(w)
    kv.append_pages(0, [0], [8192], [8192])
    for g in range(8):
        ft, kl, ids = kv.page_table(0, 0, g)
        assert (ft, kl, len(ids)) == (0, 8192, 128)
    kv.append_pages(0, [0], [1], [1])
    assert len(kv.page_table(0, 0, 0)[2]) == 129
    for g in range(1, 8):
        ft, kl, ids = kv.page_table(0, 0, g)
        exp = SG.segment_after_appends([(8192, 8192), (1, 1)], 1024, 64)
        assert (kl, ft, len(ids)) == exp == (8193, 7168, 17)
    check_pool(kv, 1, 4, 8)


def test_decode_32k_page_counts():
    w = [0] + [4096] * 7
    kv = ctx(w, seqs=31, pages=40_000)
    kv.append_pages(0, list(range(31)), [32767] * 31, [0] * 31)
    kv.append_pages(0, list(range(31)), [1] * 31, [1] * 31)
    total = 0
    for s in range(31):
        for g in range(8):
            ft, kl, ids = kv.page_table(0, s, g)
            assert kl == 32768
            assert len(ids) == (512 if g == 0 else 64)
            assert ft == (0 if g == 0 else 28672)
            total += len(ids)
    assert total == 29_760
    check_pool(kv, 1, 31, 8)


def test_fill_never_stores_out_of_window_pages():
    w = [0] + [4096] * 7
    kv = ctx(w, seqs=1, pages=10_000)
    kv.append_pages(0, [0], [122880], [0])
    for g in range(1, 8):
        ft, kl, ids = kv.page_table(0, 0, g)
        assert ft == 64 * ((122880 - 4096 + 1) // 64) and len(ids) == 64
    kv.append_pages(0, [0], [8192], [8192])
    assert len(kv.page_table(0, 0, 0)[2]) == 2048
    for g in range(1, 8):
        ft, kl, ids = kv.page_table(0, 0, g)
        assert ft == 118784 and kl == 131072 and len(ids) == 192
    assert 10_000 - kv.free_pages() == 2048 + 7 * 192


def test_random_append_sequences_match_segment_oracle():
    rng = np.random.default_rng(123)
    for trial in range(30):
        page = int(rng.choice([16, 32, 64]))
        windows = [0] + [int(x) for x in rng.integers(1, 300, size=3)]
        kv = ctx(windows, page=page, pages=5000, seqs=2)
        hist = {0: [], 1: []}
        for step in range(int(rng.integers(1, 8))):
            ids = [0, 1] if rng.random() < 0.5 else [int(rng.integers(0, 2))]
            new = [int(rng.integers(0, 200)) for _ in ids]
            nq = [int(rng.integers(0, n + 1)) for n in new]
            kv.append_pages(0, ids, new, nq)
            for s, n, q in zip(ids, new, nq):
                hist[s].append((n, q))
            for s in (0, 1):
                for g, wdw in enumerate(windows):
                    kl, ft, npg = SG.segment_after_appends(hist[s], wdw, page)
                    got = kv.page_table(0, s, g)
                    assert (got[1], got[0], len(got[2])) == (kl, ft, npg), (trial, step, s, g)
            check_pool(kv, 1, 2, 4)


def test_pool_exhaustion_is_all_or_nothing():
    kv = ctx([0, 64], page=16, pages=10, seqs=2)
    kv.append_pages(0, [0], [64], [64])          # 4 + 4 pages
    before = (kv.free_pages(), [kv.page_table(0, s, g) for s in (0, 1) for g in (0, 1)])
    with pytest.raises(S.SegKVError) as e:
        kv.append_pages(0, [0, 1], [16, 16], [1, 1])  # needs 1 + 0 (trim reuses) + 1 + 1
    assert e.value.code == S.SEGKV_E_NOMEM
    after = (kv.free_pages(), [kv.page_table(0, s, g) for s in (0, 1) for g in (0, 1)])
    assert before[0] == after[0]
    for a, b in zip(before[1], after[1]):
        assert a[0] == b[0] and a[1] == b[1] and np.array_equal(a[2], b[2])


def test_trimmed_pages_are_reused():
    kv = ctx([64], page=16, pages=6, seqs=1)
    kv.append_pages(0, [0], [64], [64])           # 4 pages
    kv.append_pages(0, [0], [64], [1])            # trims to the window, reuses freed pages
    ft, kl, ids = kv.page_table(0, 0, 0)
    assert kl == 128 and ft == 64 and len(ids) == 4
    check_pool(kv, 1, 1, 1)


def test_page_order_seed():
    a = ctx([0], page=16, pages=64, seqs=1, seed=0)
    a.append_pages(0, [0], [64], [64])
    assert a.page_table(0, 0, 0)[2].tolist() == [0, 1, 2, 3]
    b = ctx([0], page=16, pages=64, seqs=1, seed=7)
    b.append_pages(0, [0], [64], [64])
    c = ctx([0], page=16, pages=64, seqs=1, seed=7)
    c.append_pages(0, [0], [64], [64])
    assert b.page_table(0, 0, 0)[2].tolist() == c.page_table(0, 0, 0)[2].tolist()
    assert b.page_table(0, 0, 0)[2].tolist() != [0, 1, 2, 3]


def test_release_returns_every_page_across_layers():
    kv = ctx([0, 8, 0, 8], page=16, pages=200, seqs=2, layers=2)
    kv.append_pages(0, [0, 1], [40, 30], [40, 30])
    kv.append_pages(1, [0], [50], [5])
    kv.release(0)
    for l in (0, 1):
        for g in (0, 1):
            assert kv.page_table(l, 0, g)[1:] [0] == 0
            assert len(kv.page_table(l, 0, g)[2]) == 0
    check_pool(kv, 2, 2, 2)
    kv.release(1)
    assert kv.free_pages() == 200


@pytest.mark.parametrize("args,code", [
    (dict(layer=1, ids=[0], new=[1], nq=[1]), S.SEGKV_E_RANGE),
    (dict(layer=0, ids=[9], new=[1], nq=[1]), S.SEGKV_E_RANGE),
    (dict(layer=0, ids=[-1], new=[1], nq=[1]), S.SEGKV_E_RANGE),
    (dict(layer=0, ids=[0], new=[1], nq=[2]), S.SEGKV_E_INVAL),
    (dict(layer=0, ids=[0], new=[1], nq=[-1]), S.SEGKV_E_INVAL),
    (dict(layer=0, ids=[0, 0], new=[1, 1], nq=[0, 0]), S.SEGKV_E_INVAL),
    (dict(layer=0, ids=[0], new=[-3], nq=[0]), S.SEGKV_E_INVAL),
])
def test_append_errors(args, code):
    kv = ctx([0, 4], page=16, pages=10, seqs=2)
    with pytest.raises(S.SegKVError) as e:
        kv.append_pages(args["layer"], args["ids"], args["new"], args["nq"])
    assert e.value.code == code
    assert kv.free_pages() == 10


def test_empty_batches_are_no_ops():
    kv = ctx([0, 4], page=16, pages=10, seqs=2)
    kv.append_pages(0, [], [], [])
    kv.append_pages(0, [0], [0], [0])
    assert kv.free_pages() == 10


def test_growing_head_before_trimming_head_in_one_append():
    """A global head that grows is planned before a local head that trims in
    the same append; the pool only fits once the trim has returned its
    pages, so every trim of the call must land before any allocation."""
    kv = ctx([0, 16], page=16, pages=9, seqs=1)
    kv.append_pages(0, [0], [64], [64])          # 4 + 4 pages of 9
    assert kv.free_pages() == 1
    kv.append_pages(0, [0], [32], [1])           # global +2, local -4 +1
    check_pool(kv, 1, 1, 2)
    assert [len(kv.page_table(0, 0, g)[2]) for g in range(2)] == [6, 1]
    assert kv.page_table(0, 0, 1)[0] == 80
    assert kv.free_pages() == 2


def test_growing_sequence_before_trimming_sequence_in_one_batch():
    """Sequence 0 grows and sequence 1 trims in one batched append: the
    allocation for sequence 0 needs the pages sequence 1 gives back."""
    kv = ctx([16], page=16, pages=6, seqs=2)
    kv.append_pages(0, [1], [64], [64])          # 4 pages
    kv.append_pages(0, [0], [16], [16])          # 1 page
    assert kv.free_pages() == 1
    kv.append_pages(0, [0, 1], [32, 1], [32, 1])  # seq 0: +2; seq 1: -3 +1
    check_pool(kv, 1, 2, 1)
    assert len(kv.page_table(0, 0, 0)[2]) == 3
    ft, kl, ids = kv.page_table(0, 1, 0)
    assert (ft, kl, len(ids)) == (48, 65, 2)
    assert kv.free_pages() == 1
