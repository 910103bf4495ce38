"""The in-page layout of the K and V pools (page_layout.h), driven on the
CPU: every 16-byte chunk of a page has its own slot; the two rows of a pair
share each 128-byte line, one 64-byte group each; the decode's operand
loads (one row per lane of a 16-lane group, 16 bytes of it per group) read
whole lines; and the prefill and score tile copies (64 lanes, 16 bytes
each, four K rows or eight V^T rows per instruction) read 1 KiB runs."""

import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "long_context_serving_amd", "csrc")
SHAPES = [(D, P) for D in (64, 128) for P in (16, 32, 64)]


@pytest.fixture(scope="module")
def layout(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    exe = str(tmp_path_factory.mktemp("layout") / "layout_check")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", CSRC, os.path.join(HERE, "layout_check.cpp"), "-o", exe],
                   check=True)

    def get(D, P):
        out = subprocess.run([exe, str(D), str(P)], capture_output=True, text=True, check=True).stdout.split("\n")
        k = np.array(out[0].split(), dtype=np.int64).reshape(P, D // 8)
        v = np.array(out[1].split(), dtype=np.int64).reshape(D, P // 8)
        return k, v
    return get


def byte_line(elem):
    return (elem * 2) // 128


@pytest.mark.parametrize("D,P", SHAPES)
def test_every_chunk_has_its_own_slot(layout, D, P):
    k, v = layout(D, P)
    for m in (k, v):
        assert sorted(m.ravel().tolist()) == list(range(0, P * D, 8))


@pytest.mark.parametrize("D,P", SHAPES)
def test_row_pairs_share_lines(layout, D, P):
    k, v = layout(D, P)
    # K: row 2m and 2m+1, chunks 4g..4g+3 of each, fill one line, in order
    for r in range(0, P, 2):
        for g in range(D // 32):
            a, b = k[r, 4 * g:4 * g + 4], k[r + 1, 4 * g:4 * g + 4]
            assert (np.diff(a) == 8).all() and (np.diff(b) == 8).all() and b[0] == a[0] + 32
            assert a[0] % 64 == 0
    # V^T rows of 128 bytes (P = 64) pair the same way; shorter rows are row-major
    for d in range(0, D, 2):
        if P == 64:
            for g in range(2):
                a, b = v[d, 4 * g:4 * g + 4], v[d + 1, 4 * g:4 * g + 4]
                assert (np.diff(a) == 8).all() and b[0] == a[0] + 32 and a[0] % 64 == 0
        else:
            assert (v[d] == d * P + 8 * np.arange(P // 8)).all()


def whole_lines(elems):
    lines, counts = np.unique(byte_line(np.asarray(elems)), return_counts=True)
    return (counts == 8).all()


@pytest.mark.parametrize("D,P", SHAPES)
def test_decode_operand_loads_read_whole_lines(layout, D, P):
    """Lane (c16, u) of a K load of key half j, block hb, k-step kk reads
    chunk 4 kk + u of key 32 j + 8 (c16 / 4) + 4 hb + c16 % 4; of a V^T load
    of block db, chunk (32 j + 8 u) % P / 8 of channel 16 db + c16.  Keys of
    a half past the page go to the next page (its own lines)."""
    k, v = layout(D, P)
    for j in range(2):
        for hb in range(2):
            for kk in range(D // 32):
                per_page = {}
                for c16 in range(16):
                    for u in range(4):
                        key = 32 * j + 8 * (c16 // 4) + 4 * hb + c16 % 4
                        per_page.setdefault(key // P, []).append(k[key % P, 4 * kk + u])
                assert all(whole_lines(e) for e in per_page.values()), (j, hb, kk)
        for db in range(D // 16):
            per_page = {}
            for c16 in range(16):
                for u in range(4):
                    key = 32 * j + 8 * u
                    per_page.setdefault(key // P, []).append(v[16 * db + c16, (key % P) // 8])
            assert all(whole_lines(e) for e in per_page.values()), (j, db)


@pytest.mark.parametrize("D,P", SHAPES)
def test_tile_copies_read_1kib_runs(layout, D, P):
    """Slot c of a 64-key LDS tile holds K chunk (c % (D/8)) ^ swz(row) of
    row c / (D/8) (swz: row % 16 at D = 128, (row / 2) % 8 at D = 64), and
    V^T chunk (c % 8) ^ ((d / 2) % 8) of channel d = c / 8; one copy
    instruction fills 64 consecutive slots from one page (P = 64) or from
    the page holding its rows."""
    k, v = layout(D, P)
    cpr = D // 8
    kswz = (lambda r: r % 16) if cpr == 16 else (lambda r: (r // 2) % 8)
    for i in range(64 * cpr // 64):
        src = []
        for c in range(64 * i, 64 * i + 64):
            row = c // cpr
            src.append((row // P, k[row % P, (c % cpr) ^ kswz(row)]))
        pages = {p for p, _ in src}
        for p in pages:
            offs = sorted(2 * e for q, e in src if q == p)
            assert offs == list(range(offs[0], offs[0] + 16 * len(offs), 16)) and offs[0] % 128 == 0
        if P == 64:
            assert len(pages) == 1 and len(src) == 64
    if P == 64:
        for i in range(D * 8 // 64):
            offs = sorted(2 * v[c // 8, (c % 8) ^ ((c // 8 // 2) % 8)] for c in range(64 * i, 64 * i + 64))
            assert offs == list(range(offs[0], offs[0] + 1024, 16)) and offs[0] % 1024 == 0
