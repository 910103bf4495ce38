"""GPU parity of attention-mass token scores and top-k (segkv_token_scores,
segkv_topk through the C ABI) against the fp64 router oracle.

Scores: each is a sum of fp32 exponentials of score-minus-LSE terms whose
arguments carry the fp32 error of the scores and of the prefill's LSE
(~1e-5); the test allows |gpu - ref| <= 2e-3 ref + 1e-3.  Top-k is integer
work: on the same fp32 scores the GPU selection equals the oracle's exactly,
and against the fp64 scores it is a valid top-k up to the score tolerance."""

import numpy as np
import pytest

from long_context_serving_amd import runner as R
from long_context_serving_amd import segkv as S
from long_context_serving_amd import workloads as wl
from oracle import attention as A
from oracle import rope as RP
from oracle import router as RT

from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load_library()


def gpu_scores(w, x, split=None, seed=None, deltas=None, style=0):
    """Prefill (default work split) for the LSE, then the scores pass with
    the given split knob."""
    import torch
    dev = R.to_device(w, x)
    run = R.WorkloadRun(w, dev, page_order_seed=seed, deltas=deltas, rope_style=style)
    try:
        run.load()
        o, lse = run.prefill()
        if split is not None:
            run.ctx.set_tuning(S.TUNE_PREFILL_SPLIT_TILES, split)
        sc = run.ctx.token_scores(0, run.seq_ids, w.q_lens, dev.q, lse)
        torch.cuda.synchronize()
        return sc.cpu().numpy().astype(np.float64)
    finally:
        run.close()


def ref_scores(w, x, deltas=None, style=0):
    out = []
    for b in range(w.n_seqs):
        q = A.bf16_bits_to_f64(x.q[x.cu_q[b]:x.cu_q[b + 1]])
        if deltas is not None:
            for g in range(w.num_kv_heads):
                hs = slice(g * w.group, (g + 1) * w.group)
                q[:, hs] = RP.relocate_queries(q[:, hs], deltas[b][g], 10000.0, style)
        k = A.bf16_bits_to_f64(x.k[x.cu_kv[b]:x.cu_kv[b + 1]])
        out.append(RT.token_scores(q, k, w.windows, w.scale))
    return np.concatenate(out) if out else np.zeros(0)


def check_scores(got, ref):
    err = np.abs(got - ref) - 2e-3 * np.abs(ref)
    say(f"  scores n={len(ref)} max|d|={np.abs(got - ref).max() if len(ref) else 0:.3e} max ref {ref.max() if len(ref) else 0:.3f}")
    assert np.all(np.isfinite(got))
    assert err.max() <= 1e-3 if len(ref) else True


@pytest.mark.parametrize("case", [
    # kv_lens, q_lens, hq, hkv, d, page, windows
    ((512,), (512,), 4, 4, 64, 16, (0, 64, 64, 64)),
    ((700,), (700,), 16, 4, 128, 64, (0, 100, 300, 64)),
    ((2000,), (333,), 8, 8, 128, 32, (0, 1000, 10, 77, 0, 5, 64, 2000)),
    ((900, 17, 300), (900, 5, 300), 16, 4, 128, 64, (0, 64, 128, 33)),
    ((640,), (640,), 12, 4, 64, 32, (13, 0, 200, 640)),
    ((600,), (600,), 16, 1, 128, 64, (0,)),  # G = 16
])
def test_scores_match_oracle(case):
    kv, q, hq, hkv, d, p, windows = case
    w = wl.small_workload("scores", kv, q, hq, hkv, d, p, windows, seed=sum(kv) + d)
    x = wl.make_inputs(w)
    say(f"scores kv={kv} q={q} hq={hq} hkv={hkv} d={d} p={p} W={windows}")
    check_scores(gpu_scores(w, x), ref_scores(w, x))


def test_scores_with_relocated_queries():
    w = wl.small_workload("scores_rope", (800,), (800,), 16, 4, 128, 64, (0, 100, 300, 64), seed=4)
    x = wl.make_inputs(w)
    deltas = [[0, 4096, 77, 123457]]
    check_scores(gpu_scores(w, x, deltas=deltas, style=1), ref_scores(w, x, deltas=deltas, style=1))


def test_scores_are_bitwise_independent_of_split_and_page_order():
    w = wl.small_workload("scores_det", (1500, 700), (1500, 300), 8, 2, 128, 64, (0, 256), seed=12)
    x = wl.make_inputs(w)
    a = gpu_scores(w, x)
    for split, seed in ((2, None), (5, 999), (1 << 30, 0)):
        assert np.array_equal(a, gpu_scores(w, x, split=split, seed=seed))
    check_scores(a, ref_scores(w, x))


def test_scores_full_size_headline():
    w = wl.MISTRAL7B_PREFILL
    x = wl.make_inputs(w)
    say(f"scores {w.name}")
    got = gpu_scores(w, x)
    ref = ref_scores(w, x)
    check_scores(got, ref)
    assert abs(got.sum() - ref.sum()) <= 1e-3 * ref.sum()


def run_topk(counts, scores, ks):
    import torch
    kv = S.SegKV(1, 2, 2, 64, 16, 1, 4, [0, 0])
    try:
        out = kv.topk(counts, torch.from_numpy(np.ascontiguousarray(scores, np.float32)).cuda(), ks)
        torch.cuda.synchronize()
        return out.cpu().numpy()
    finally:
        kv.close()


def split_out(out, ks):
    offs = np.concatenate([[0], np.cumsum(ks)])
    return [out[offs[i]:offs[i + 1]] for i in range(len(ks))]


@pytest.mark.parametrize("counts,ks", [((10,), (3,)), ((1000, 1, 5000, 7), (1, 1, 2500, 0)), ((4096,), (4096,)),
                                       ((200_000, 3333), (50_000, 17)), ((1025, 2047), (512, 1)),
                                       # either side of the largest sequence kept in registers (8192 keys)
                                       ((8192, 8193), (4096, 8192)), ((8192, 8193), (1, 1))])
def test_topk_matches_oracle_exactly(counts, ks):
    rng = np.random.default_rng(sum(counts))
    s = rng.exponential(1.0, size=sum(counts)).astype(np.float32)
    s[::97] = s[1]  # many ties
    if len(s) > 3:
        s[3] = 0.0
    got = split_out(run_topk(counts, s, ks), ks)
    at = 0
    for n, k, g in zip(counts, ks, got):
        want = RT.top_k(s[at:at + n].astype(np.float64), k)
        assert np.array_equal(g, want), (n, k)
        at += n


def test_topk_of_equal_and_nearly_equal_scores():
    # all keys equal (the lowest indices win), and keys equal but for their
    # lowest mantissa bits
    counts, ks = (5000, 3000, 7), (1234, 2999, 3)
    s = np.concatenate([np.full(5000, 0.75, np.float32),
                        (np.float32(3.0).view(np.uint32) + np.arange(3000, dtype=np.uint32) % 5).view(np.float32),
                        np.full(7, 2.0, np.float32)])
    got = split_out(run_topk(counts, s, ks), ks)
    at = 0
    for n, k, g in zip(counts, ks, got):
        assert np.array_equal(g, RT.top_k(s[at:at + n].astype(np.float64), k)), (n, k)
        at += n


def test_topk_of_gpu_scores_is_a_valid_selection():
    import torch
    w = wl.small_workload("route", (2000, 700), (2000, 700), 16, 4, 128, 64, (0, 64, 128, 33), seed=8)
    x = wl.make_inputs(w)
    got = gpu_scores(w, x)
    ref = ref_scores(w, x)
    ks = (500, 70)
    sel = split_out(run_topk(w.q_lens, got, ks), ks)
    at = 0
    for n, k, g in zip(w.q_lens, ks, sel):
        assert np.array_equal(g, RT.top_k(got[at:at + n].astype(np.float32).astype(np.float64), k))
        r = ref[at:at + n]
        chosen = np.zeros(n, bool)
        chosen[g] = True
        tol = 2e-3 * r.max() + 1e-3
        assert r[chosen].min() >= r[~chosen].max() - 2 * tol
        at += n
