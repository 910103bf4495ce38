"""GPU parity of the head-decomposition merge (segkv_merge, through the C ABI)
against the fp64 merge oracle on the same seeded inputs.

Selected pairs must come back bit for bit.  Merged pairs are one fp32
evaluation rounded once to bf16: |o - ref| <= 2^-8 max(1, |ref|) and |lse -
ref| <= 1e-5 (1 + |ref|), far inside the 2e-2 / 1e-3 parity bar."""

import dataclasses

import numpy as np
import pytest

from long_context_serving_amd import segkv as S
from long_context_serving_amd import workloads as wl
from oracle import attention as A
from oracle import merge as MO

from gpu_helpers import compare, gpu_run, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load_library()


def ctx_for(hq, d, hkv=None):
    hkv = hkv or hq
    return S.SegKV(1, hq, hkv, d, 64, 1, 4, [0] * hkv)


def to_dev(mi):
    import torch
    return (S.bf16_tensor(mi.o_a), torch.from_numpy(mi.lse_a).cuda(), S.bf16_tensor(mi.o_b),
            torch.from_numpy(mi.lse_b).cuda(), torch.from_numpy(mi.mode).cuda())


def check(mi, o_bits, lse, rows=None):
    sel = slice(None) if rows is None else rows
    mode = mi.mode[sel]
    ref_o, ref_l = MO.head_decomposition_merge(A.bf16_bits_to_f64(mi.o_a[sel]), mi.lse_a[sel].astype(np.float64),
                                               A.bf16_bits_to_f64(mi.o_b[sel]), mi.lse_b[sel].astype(np.float64),
                                               np.minimum(mode, 2))
    ob = o_bits[sel]
    ta, tb = mode == 0, mode == 1
    assert np.array_equal(ob[ta], mi.o_a[sel][ta]) and np.array_equal(lse[sel][ta], mi.lse_a[sel][ta])
    assert np.array_equal(ob[tb], mi.o_b[sel][tb]) and np.array_equal(lse[sel][tb], mi.lse_b[sel][tb])
    mg = mode >= 2
    if mg.any():
        go = A.bf16_bits_to_f64(ob[mg])
        ro = ref_o[mg]
        gl, rl = lse[sel][mg].astype(np.float64), ref_l[mg]
        empty = np.isneginf(rl)
        assert np.all(np.isneginf(gl[empty])) and np.all(go[empty] == 0)
        do = np.abs(go - ro) / np.maximum(1.0, np.abs(ro))
        dl = np.abs(gl[~empty] - rl[~empty]) / (1.0 + np.abs(rl[~empty]))
        say(f"  merged pairs {int(mg.sum())}: max rel |do| {do.max():.3e} max rel |dlse| {dl.max() if dl.size else 0:.3e}")
        assert do.max() <= 2.0 ** -8
        assert dl.size == 0 or dl.max() <= 1e-5


@pytest.mark.parametrize("rows,hq,d,empty", [(1, 8, 128, 0.0), (37, 12, 64, 0.2), (1000, 32, 128, 0.1),
                                              (3001, 4, 64, 0.5)])
def test_merge_random_partials_match_oracle(rows, hq, d, empty):
    import torch
    mw = wl.MergeWorkload("m", rows, hq, hq // 2 if hq > 1 else 1, d, window=0, tail=0, query_rows=0,
                          boundary_every=rows + 1, dirty_frac=0.0, seed=rows + d, empty_frac=empty)
    mi = wl.make_merge_inputs(mw)
    rng = np.random.default_rng(rows)
    mi.mode = rng.integers(0, 4, size=mi.mode.shape).astype(np.uint8)  # 3 = merge too
    both = rng.random(mi.mode.shape) < 0.05
    mi.lse_a[both] = -np.inf
    mi.lse_b[both] = -np.inf
    mi.lse_b[0, 0], mi.lse_a[0, 0] = 80.0, -80.0  # extreme gap
    say(f"merge rows={rows} hq={hq} d={d} empty={empty}")
    kv = ctx_for(hq, d)
    o, lse = kv.merge(*to_dev(mi))
    torch.cuda.synchronize()
    check(mi, S.bf16_bits(o), lse.cpu().numpy())
    kv.close()


def test_merge_in_place_and_without_lse():
    import torch
    mw = wl.MergeWorkload("m", 777, 16, 4, 128, window=300, tail=100, query_rows=10, boundary_every=128,
                          dirty_frac=0.05, seed=9, empty_frac=0.05)
    mi = wl.make_merge_inputs(mw)
    kv = ctx_for(16, 128, 4)
    oa, la, ob, lb, md = to_dev(mi)
    o_ref, l_ref = kv.merge(oa, la, ob, lb, md)
    o_nl, l_nl = kv.merge(oa, la, ob, lb, md, want_lse=False)
    assert l_nl is None
    kv.merge(oa, la, ob, lb, md, o=ob, lse=lb)  # in place over B
    torch.cuda.synchronize()
    assert torch.equal(o_ref, ob) and torch.equal(l_ref, lb) and torch.equal(o_ref, o_nl)
    check(mi, S.bf16_bits(o_ref), l_ref.cpu().numpy())
    kv.close()


def test_merge_full_size_sampled_rows():
    """The 128K-document merge in the launch configuration the benchmark
    times, checked on sampled rows (boundaries of every region, random)."""
    import torch
    mw = wl.MERGE_128K
    mi = wl.make_merge_inputs(mw)
    kv = ctx_for(mw.num_q_heads, mw.head_dim, mw.num_kv_heads)
    say(f"merge {mw.name} rows={mw.rows}")
    o, lse = kv.merge(*to_dev(mi))
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    edges = [0, 1, mw.window - 2, mw.window - 1, 127, 128, 129, mw.rows - mw.tail - 1, mw.rows - mw.tail,
             mw.rows - 1]
    rows = np.unique(np.concatenate([edges, rng.integers(0, mw.rows, 3000)]))
    o_bits = S.bf16_bits(o[torch.from_numpy(rows).cuda()])
    l = lse[torch.from_numpy(rows).cuda()].cpu().numpy()
    sub = wl.MergeInputs(mi.o_a[rows], mi.lse_a[rows], mi.o_b[rows], mi.lse_b[rows], mi.mode[rows])
    check(sub, o_bits, l)
    kv.close()


def test_decomposition_with_prefill_outputs_reproduces_the_request():
    """A request = a prefix of a tokens + a document of n tokens, one prefill
    call over two sequences: the whole request (online B: the document's
    rows at their live positions) and the document alone (offline A).  Global
    heads and protected rows (here also every local row that sees prefix
    keys) take B, the rest A; the merged output is the request's attention."""
    import torch
    from long_context_serving_amd import runner as R
    a, n, hq, hkv, d = 200, 700, 16, 4, 128
    windows = (0, 64, 128, 300)
    w = wl.small_workload("decomp", (a + n, n), (n, n), hq, hkv, d, 64, windows, seed=5)
    x = wl.make_inputs(w)
    k, v = x.k.copy(), x.v.copy()
    k[a + n:], v[a + n:] = x.k[a:a + n], x.v[a:a + n]  # the document alone holds the same tokens
    q = np.concatenate([x.q[:n], x.q[:n]])           # and the same query rows
    x = dataclasses.replace(x, q=q, k=k, v=v)
    o_bits, lse = gpu_run(w, x)
    compare(w, x, o_bits, lse)
    mode = np.full((n, hq), wl.TAKE_A, np.uint8)
    local = np.array([windows[h // (hq // hkv)] > 0 for h in range(hq)])
    wmax = max(windows)
    mode[: wmax - 1, :] = wl.TAKE_B                  # local rows that also see prefix keys
    mode[::128, :] = wl.TAKE_B
    mode[:, ~local] = wl.TAKE_B
    dev = lambda t: torch.from_numpy(np.ascontiguousarray(t)).cuda()
    kv = ctx_for(hq, d, hkv)
    o, l = kv.merge(S.bf16_tensor(o_bits[n:]), dev(lse[n:].astype(np.float32)), S.bf16_tensor(o_bits[:n]),
                    dev(lse[:n].astype(np.float32)), dev(mode))
    torch.cuda.synchronize()
    ref_o, ref_l = A.attend_sequence(A.bf16_bits_to_f64(x.q[:n]), A.bf16_bits_to_f64(x.k[:a + n]),
                                     A.bf16_bits_to_f64(x.v[:a + n]), windows, w.scale)
    go = A.bf16_bits_to_f64(S.bf16_bits(o))
    gl = l.cpu().numpy().astype(np.float64)
    say(f"  decomposed vs request: max|do|={np.abs(go - ref_o).max():.3e} max|dlse|={np.abs(gl - ref_l).max():.3e}")
    assert np.abs(go - ref_o).max() <= 2e-2 and np.abs(gl - ref_l).max() <= 1e-3
    # the offline output alone misses the prefix keys on the boundary rows
    assert np.abs(lse[n:][: wmax - 1][:, local] - ref_l[: wmax - 1][:, local]).max() > 1e-2
    kv.close()


def test_merge_timing_and_errors():
    import torch
    kv = ctx_for(8, 64)
    mw = wl.MergeWorkload("m", 64, 8, 8, 64, 0, 0, 0, 65, 0.0, seed=1)
    oa, la, ob, lb, md = to_dev(wl.make_merge_inputs(mw))
    kv.set_timing(True, [S.KERNEL_MERGE])
    kv.merge(oa, la, ob, lb, md)
    ms, cnt = kv.read_timing(S.KERNEL_MERGE)
    assert cnt == 1 and ms > 0
    kv.set_timing(False)
    lib = kv._lib
    assert lib.segkv_merge(kv._h, 64, oa.data_ptr() + 2, la.data_ptr(), ob.data_ptr(), lb.data_ptr(),
                           md.data_ptr(), oa.data_ptr(), None) == S.SEGKV_E_INVAL
    assert lib.segkv_merge(kv._h, 64, oa.data_ptr(), la.data_ptr(), ob.data_ptr(), lb.data_ptr(),
                           None, oa.data_ptr(), None) == S.SEGKV_E_INVAL
    assert lib.segkv_merge(kv._h, 0, None, None, None, None, None, None, None) == S.SEGKV_OK
    with pytest.raises(ValueError):
        kv.merge(oa, la, ob, lb, md[:3])
    torch.cuda.synchronize()
    kv.close()
