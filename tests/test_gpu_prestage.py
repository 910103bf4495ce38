"""Prefill tables staged by the append.

An append whose queries form a prefill chunk puts the tables of that
prefill on the device inside its own scatter launch; the prefill call uses
them when the tables it builds are the same byte for byte and nothing has
written the device tables since, and uploads its own otherwise.  Both paths
must give the oracle's results, and the same bits."""

import numpy as np
import pytest

from long_context_serving_amd import runner as R
from long_context_serving_amd import segkv as S
from long_context_serving_amd import workloads as wl

from gpu_helpers import compare, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load_library()


def uploads(ctx):
    return ctx.read_timing(S.KERNEL_UPLOAD)[1]


def test_prefill_after_its_append_uses_the_staged_tables():
    import torch
    w = wl.small_workload("prestage", (900, 500, 70), (300, 500, 70), 16, 4, 128, 64, (0, 64, 200, 1000), seed=51)
    x = wl.make_inputs(w)
    say(f"prefill {w.name} kv={w.kv_lens} q={w.q_lens}")
    run = R.WorkloadRun(w, R.to_device(w, x))
    try:
        run.ctx.set_timing(True, [S.KERNEL_UPLOAD])
        run.load()
        o1, l1 = run.prefill()
        torch.cuda.synchronize()
        assert uploads(run.ctx) == 0  # the append's scatter launch carried the tables
        o2, l2 = run.prefill()  # same call again: the staged tables were used up
        torch.cuda.synchronize()
        assert uploads(run.ctx) == 1
        b1, b2 = S.bf16_bits(o1), S.bf16_bits(o2)
        assert np.array_equal(b1, b2) and np.array_equal(l1.cpu().numpy(), l2.cpu().numpy())
        compare(w, x, b1, l1.cpu().numpy().astype(np.float64))
        run.ctx.set_timing(False)
    finally:
        run.close()


def test_staged_tables_repeat_across_steps():
    # release, append and prefill again on one context, as a serving loop does
    import torch
    w = wl.small_workload("prestage_loop", (1500,), (600,), 8, 2, 128, 64, (0, 256), seed=52)
    x = wl.make_inputs(w)
    say(f"prefill {w.name} kv={w.kv_lens} q={w.q_lens}")
    run = R.WorkloadRun(w, R.to_device(w, x))
    try:
        run.ctx.set_timing(True, [S.KERNEL_UPLOAD])
        outs = []
        for _ in range(3):
            run.reset()
            run.load()
            o, l = run.prefill()
            torch.cuda.synchronize()
            outs.append((S.bf16_bits(o), l.cpu().numpy()))
        assert uploads(run.ctx) == 0
        for o, l in outs[1:]:
            assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])
        compare(w, x, outs[0][0], outs[0][1].astype(np.float64))
        run.ctx.set_timing(False)
    finally:
        run.close()


def test_tables_staged_for_another_layer_are_not_used():
    # layer 1's append stages its own tables after layer 0's: the layer-0
    # prefill must see the difference and upload, the layer-1 one need not
    import torch
    hq, hkv, d, p = 8, 2, 128, 64
    win = [(0, 128), (0, 0)]
    w0 = wl.small_workload("prestage_l0", (700, 260), (300, 260), hq, hkv, d, p, win[0], seed=53)
    w1 = wl.small_workload("prestage_l1", (700, 260), (300, 260), hq, hkv, d, p, win[1], seed=53)
    x = wl.make_inputs(w0)
    dev = R.to_device(w0, x)
    say(f"prefill two layers kv={w0.kv_lens} q={w0.q_lens} windows={win}")
    ctx = S.SegKV(2, hq, hkv, d, p, 2, 2 * R.pages_for(w1), win[0] + win[1], softmax_scale=w0.scale)
    try:
        ctx.set_timing(True, [S.KERNEL_UPLOAD])
        ids = [0, 1]
        fill = w0.fill_lens()
        for layer in (0, 1):
            ctx.append_pages(layer, ids, fill, [0, 0], dev.k_fill, dev.v_fill)
            ctx.append_pages(layer, ids, w0.q_lens, w0.q_lens, dev.k_q, dev.v_q)
        o0, l0 = ctx.prefill(0, ids, w0.q_lens, dev.q)
        torch.cuda.synchronize()
        assert uploads(ctx) == 1
        o1, l1 = ctx.prefill(1, ids, w1.q_lens, dev.q)
        torch.cuda.synchronize()
        assert uploads(ctx) == 2  # the layer-0 upload replaced layer 1's staged tables
        compare(w0, x, S.bf16_bits(o0), l0.cpu().numpy().astype(np.float64))
        compare(w1, x, S.bf16_bits(o1), l1.cpu().numpy().astype(np.float64), windows=win[1])
        for s in ids:  # the other order: layer 1's tables are current
            ctx.release(s)
        for layer in (0, 1):
            ctx.append_pages(layer, ids, fill, [0, 0], dev.k_fill, dev.v_fill)
            ctx.append_pages(layer, ids, w0.q_lens, w0.q_lens, dev.k_q, dev.v_q)
        o1b, l1b = ctx.prefill(1, ids, w1.q_lens, dev.q)
        torch.cuda.synchronize()
        assert uploads(ctx) == 2
        assert np.array_equal(S.bf16_bits(o1b), S.bf16_bits(o1))
        ctx.set_timing(False)
    finally:
        ctx.close()


def test_relocation_set_after_the_append_is_not_missed():
    # offsets set between the append and the prefill change the segment
    # tables: the staged ones no longer match and the prefill uploads its own
    import torch
    w = wl.small_workload("prestage_rope", (900, 400), (300, 400), 8, 2, 128, 64, (0, 256), seed=54)
    x = wl.make_inputs(w)
    rope = dict(deltas=[[0, 4096], [0, 77]])
    say(f"prefill {w.name} kv={w.kv_lens} q={w.q_lens} rope={rope}")
    run = R.WorkloadRun(w, R.to_device(w, x), deltas=rope["deltas"])
    try:
        run.ctx.set_timing(True, [S.KERNEL_UPLOAD])
        run.load()  # appends, then sets the offsets
        o, l = run.prefill()
        torch.cuda.synchronize()
        assert uploads(run.ctx) == 1
        compare(w, x, S.bf16_bits(o), l.cpu().numpy().astype(np.float64), rope=rope)
        run.ctx.set_timing(False)
    finally:
        run.close()
