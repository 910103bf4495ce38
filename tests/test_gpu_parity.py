"""GPU parity: libsegkv (through the C ABI) against the fp64 oracle on the
same seeded inputs.  bf16 outputs within max-abs 2e-2 and LSE within 1e-3
of the unrounded oracle; integer page state exactly."""

import numpy as np
import pytest

from long_context_serving_amd import segkv as S
from long_context_serving_amd import workloads as wl

from gpu_helpers import compare, gpu_run, sample_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load_library()


def small(name, kv, q, hq, hkv, d, p, windows, seed):
    return wl.small_workload(name, kv, q, hq, hkv, d, p, windows, seed)


def test_tiny_mha_all_rows():
    w = wl.TINY_MHA
    x = wl.make_inputs(w)
    o, lse = gpu_run(w, x)
    compare(w, x, o, lse)


@pytest.mark.parametrize("case", [
    # kv_lens, q_lens, hq, hkv, d, page, windows
    ((200,), (200,), 4, 4, 64, 16, (0, 1, 7, 64)),
    ((333,), (333,), 8, 2, 128, 64, (0, 100)),
    ((257,), (257,), 8, 1, 64, 32, (0,)),
    ((130,), (130,), 16, 2, 128, 16, (129, 130)),
    ((500,), (500,), 32, 4, 128, 64, (0, 64, 1000, 1)),
    ((300,), (300,), 24, 8, 64, 32, (0, 5, 63, 64, 65, 299, 300, 600)),
    ((640,), (640,), 12, 4, 128, 16, (13, 0, 200, 640)),    # G = 3 does not divide the 128-row tile
    ((600,), (600,), 16, 1, 128, 64, (0,)),                 # G = 16, the largest group: 16 positions per item
    ((450,), (450,), 32, 2, 64, 64, (0, 100)),               # G = 16 with D = 64 on 64-token pages
])
def test_prefill_shapes(case):
    kv, q, hq, hkv, d, p, windows = case
    w = small("shape", kv, q, hq, hkv, d, p, windows, seed=sum(kv) + hq + d + p)
    x = wl.make_inputs(w)
    o, lse = gpu_run(w, x)
    compare(w, x, o, lse)


@pytest.mark.parametrize("case", [
    ((700,), (96,), 8, 2, 128, 64, (0, 130)),            # chunk after a cache fill
    ((1000,), (1,), 8, 8, 64, 16, (0, 7, 100, 1000, 3, 1, 999, 2)),
    ((2000,), (333,), 4, 4, 128, 32, (0, 1000, 10, 77)),  # window not a multiple of the page
    ((900, 17, 64, 500), (900, 5, 64, 1), 16, 4, 128, 64, (0, 64, 128, 33)),  # varlen batch
    ((40, 300), (0, 300), 4, 2, 64, 16, (0, 9)),          # one sequence without queries
])
def test_prefill_chunked_and_varlen(case):
    kv, q, hq, hkv, d, p, windows = case
    w = small("chunk", kv, q, hq, hkv, d, p, windows, seed=sum(kv) * 7 + sum(q))
    x = wl.make_inputs(w)
    o, lse = gpu_run(w, x)
    compare(w, x, o, lse)


def test_prefill_peaky_softmax_and_planted_key():
    w = small("peaky", (600,), (600,), 8, 2, 128, 64, (0, 100), seed=77)
    x = wl.make_inputs(w, q_scale=3.0)
    # plant one key that dominates every row that can see it, late in the sequence
    k = x.k.view(np.uint16)
    q0 = x.q[550, 0].copy()
    k[540, 0] = q0  # score of row 550 with key 540 = |q|^2 * scale, far above the rest
    o, lse = gpu_run(w, x)
    compare(w, x, o, lse)


def test_prefill_bitwise_deterministic_and_page_order_invariant():
    w = small("det", (700,), (700,), 16, 4, 128, 16, (0, 64, 200, 700), seed=5)
    x = wl.make_inputs(w)
    (o1, l1), (o2, l2) = gpu_run(w, x, seed=1, repeat=2)
    o3, l3 = gpu_run(w, x, seed=12345)
    o4, l4 = gpu_run(w, x, seed=0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)
    assert np.array_equal(o1, o4) and np.array_equal(l1, l4)
    compare(w, x, o1, l1)


def test_wide_local_window_equals_global_on_gpu():
    w = small("wide", (500,), (500,), 8, 2, 128, 64, (0, 0), seed=9)
    x = wl.make_inputs(w)
    og, lg = gpu_run(w, x, windows=(0, 0))
    ol, ll = gpu_run(w, x, windows=(500, 10_000))
    assert np.array_equal(og, ol) and np.array_equal(lg, ll)


@pytest.mark.parametrize("split", [1, 3, 8])
def test_prefill_split_kv_matches_oracle(split):
    w = small("split", (1500, 700), (1500, 300), 8, 2, 128, 64, (0, 256), seed=31)
    x = wl.make_inputs(w)
    o, lse = gpu_run(w, x, split_tiles=split)
    compare(w, x, o, lse)


# ---------------------------------------------------------------- decode

def decode_workload(name, n, kv, hq, hkv, d, p, windows, seed):
    return wl.Workload(name, (kv,) * n if isinstance(kv, int) else tuple(kv), (1,) * (n if isinstance(kv, int) else len(kv)),
                       hq, hkv, d, p, tuple(windows), seed, decode=True)


@pytest.mark.parametrize("case", [
    (5, 3000, 64, 8, 128, 64, (0, 512, 512, 512, 512, 512, 512, 512), 16),
    (3, (1, 63, 65), 16, 16, 64, 16, (0, 1, 2, 7, 64, 0, 5, 9, 10, 11, 12, 13, 14, 15, 16, 17), 4),
    (4, (100, 1000, 2049, 77), 32, 2, 128, 32, (0, 300), 3),
    (2, 5000, 16, 1, 64, 64, (0,), 1),
    (2, 4097, 64, 4, 128, 16, (4096, 0, 100, 1), None),
    (3, (900, 64, 2000), 48, 2, 128, 64, (0, 200), 8),      # G = 24: blocks of 16 and 8 query heads
    (2, 3000, 64, 1, 64, 32, (0,), None),                   # G = 64 (one KV head): four blocks
])
def test_decode_shapes(case):
    n, kv, hq, hkv, d, p, windows, pps = case
    w = decode_workload("dec", n, kv, hq, hkv, d, p, windows, seed=n * 13 + d)
    x = wl.make_inputs(w)
    o, lse = gpu_run(w, x, mode="decode", pps=pps)
    compare(w, x, o, lse)


def test_decode_matches_prefill_of_last_token():
    w = decode_workload("dec_vs_pf", 3, (700, 1200, 64), 16, 4, 128, 64, (0, 100, 300, 5), seed=3)
    x = wl.make_inputs(w)
    od, ld = gpu_run(w, x, mode="decode")
    op, lp = gpu_run(w, x, mode="prefill")
    a = np.abs(od.view(np.uint16).astype(np.int64) - op.view(np.uint16).astype(np.int64))
    compare(w, x, od, ld)
    compare(w, x, op, lp)
    say(f"  decode vs prefill max ulp-ish diff {int(a.max())}")


# ------------------------------------------------------- errors on device

def test_device_context_errors():
    import torch
    w = small("err", (64,), (64,), 4, 2, 64, 16, (0, 16), seed=1)
    x = wl.make_inputs(w)
    from long_context_serving_amd import runner as R
    dev = R.to_device(w, x)
    run = R.WorkloadRun(w, dev, num_pages=9)
    # 64 tokens need 4 pages per head: 8 pages fit, the next append of 64 does not
    run.load()
    free = run.ctx.free_pages()
    with pytest.raises(S.SegKVError) as e:
        run.ctx.append_pages(0, [0], [64], [64], dev.k_q, dev.v_q)
    assert e.value.code == S.SEGKV_E_NOMEM and run.ctx.free_pages() == free
    with pytest.raises(S.SegKVError) as e:   # queries reach before the declared pending query
        run.ctx.prefill(0, [0], [65], torch.zeros((65, 4, 64), dtype=torch.bfloat16, device="cuda"))
    assert e.value.code == S.SEGKV_E_INVAL
    run.ctx.append_pages(0, [0], [0], [0])     # n_query = 0: nothing pending any more
    with pytest.raises(S.SegKVError) as e:
        run.ctx.prefill(0, [0], [64], dev.q)
    assert e.value.code == S.SEGKV_E_INVAL
    with pytest.raises(S.SegKVError) as e:
        run.ctx.decode(0, [0], dev.q[:1])
    assert e.value.code == S.SEGKV_E_INVAL
    with pytest.raises(S.SegKVError) as e:
        run.ctx.prefill(0, [3], [1], dev.q[:1])
    assert e.value.code == S.SEGKV_E_RANGE
    run.close()


def test_prefill_work_order_does_not_change_results():
    w = small("order", (2000, 900, 64), (2000, 900, 64), 16, 4, 128, 64, (0, 300, 64, 1000), seed=41)
    x = wl.make_inputs(w)
    from long_context_serving_amd import runner as R
    import torch
    outs = []
    for order, split in ((0, 0), (1, 0), (0, 1 << 30), (1, 1 << 30)):
        run = R.WorkloadRun(w, R.to_device(w, x))
        run.ctx.set_tuning(S.TUNE_PREFILL_ORDER, order)
        run.ctx.set_tuning(S.TUNE_PREFILL_SPLIT_TILES, split)
        run.load()
        o, lse = run.prefill()
        torch.cuda.synchronize()
        outs.append((S.bf16_bits(o), lse.cpu().numpy().astype(np.float64)))
        run.close()
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[2][0], outs[3][0]) and np.array_equal(outs[2][1], outs[3][1])
    for o, l in outs:
        compare(w, x, o, l)


def test_decode_repeated_calls_agree():
    # many parts per segment: exercises the arrival counters across calls
    w = decode_workload("dec_rep", 4, (5000, 300, 2500, 64), 32, 4, 128, 64, (0, 1000, 64, 0), seed=8)
    x = wl.make_inputs(w)
    (o1, l1), (o2, l2), (o3, l3) = gpu_run(w, x, mode="decode", pps=2, repeat=3)
    assert np.array_equal(o1, o2) and np.array_equal(o1, o3)
    assert np.array_equal(l1, l2) and np.array_equal(l1, l3)
    compare(w, x, o1, l1)


def test_kernel_timing_mask():
    from long_context_serving_amd import runner as R
    w = small("timing", (700,), (700,), 8, 2, 128, 64, (0, 100), seed=2)
    x = wl.make_inputs(w)
    run = R.WorkloadRun(w, R.to_device(w, x))
    run.ctx.set_timing(True, [S.KERNEL_PREFILL])
    run.load()
    run.prefill()
    ms, n = run.ctx.read_timing(S.KERNEL_PREFILL)
    assert n == 1 and ms > 0
    assert run.ctx.read_timing(S.KERNEL_SCATTER) == (0.0, 0)
    run.ctx.set_timing(False)
    with pytest.raises(S.SegKVError):
        run.ctx._check(run.ctx._lib.segkv_set_timing(run.ctx._h, 1 << 9))
    run.close()


@pytest.mark.parametrize("case", [
    # many one-tile items (the work queue's producer falls behind) mixed with long ones
    (tuple(range(1, 61)), tuple(range(1, 61)), 8, 2, 128, 64, (0, 16)),
    (tuple(3 + (7 * i) % 50 for i in range(90)) + (1500,), tuple(min(1 + (3 * i) % 5, 3 + (7 * i) % 50) for i in range(90)) + (700,),
     16, 4, 64, 16, (0, 5, 64, 300)),
    ((1,) * 40 + (2000,), (1,) * 40 + (2000,), 4, 1, 128, 32, (0,)),
])
def test_prefill_many_short_items(case):
    kv, q, hq, hkv, d, p, windows = case
    w = small("short_items", kv, q, hq, hkv, d, p, windows, seed=len(kv) + d)
    x = wl.make_inputs(w)
    o, lse = gpu_run(w, x)
    rows = [sample_rows(w, b, n_random=64) for b in range(w.n_seqs)]
    compare(w, x, o, lse, rows_per_seq=rows)
