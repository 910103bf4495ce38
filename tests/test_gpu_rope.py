"""GPU parity of query-side RoPE relocation: libsegkv with per-(sequence, KV
head) offsets, through the C ABI, against the fp64 relocation oracle on the
same seeded inputs (bf16 outputs within max-abs 2e-2, LSE within 1e-3)."""

import dataclasses

import numpy as np
import pytest

from long_context_serving_amd import segkv as S
from long_context_serving_amd import workloads as wl
from oracle import attention as A
from oracle import rope as RP

from gpu_helpers import PREFILL_KERNEL, compare, gpu_run, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load_library()


@pytest.mark.parametrize("case", [
    # kv_lens, q_lens, hq, hkv, d, page, windows, style, rope_dims, deltas[seq][kv head]
    ((700,), (700,), 16, 4, 128, 64, (0, 100, 300, 64), 0, 0, [[4096, 0, 123457, -77]]),
    ((333,), (333,), 8, 2, 64, 16, (0, 40), 1, 32, [[1000, 5]]),
    ((900, 17, 300), (900, 5, 300), 16, 4, 128, 32, (0, 64, 128, 33), 0, 64,
     [[1, 2, 3, 4], [0, 0, 0, 0], [500000, 0, 7, 7]]),
    ((2000,), (333,), 8, 8, 128, 64, (0, 1000, 10, 77, 0, 5, 64, 2000), 1, 0,
     [[8192, 8192, 8192, 8192, 0, 1, 2, 3]]),
    ((640,), (640,), 12, 4, 64, 32, (13, 0, 200, 640), 0, 16, [[31, 32000, 0, -1]]),
])
def test_prefill_relocated_matches_oracle(case):
    kv, q, hq, hkv, d, p, windows, style, dims, deltas = case
    w = wl.small_workload("rope", kv, q, hq, hkv, d, p, windows, seed=sum(kv) + 3 * d + style)
    x = wl.make_inputs(w)
    rope = dict(deltas=deltas, style=style, dims=dims)
    o, lse = gpu_run(w, x, rope=rope)
    compare(w, x, o, lse, rope=rope)


@pytest.mark.parametrize("split", [2, 5])
def test_prefill_relocated_split_kv(split):
    w = wl.small_workload("rope_split", (1500, 700), (1500, 300), 8, 2, 128, 64, (0, 256), seed=12)
    x = wl.make_inputs(w)
    rope = dict(deltas=[[100, 65536], [-3, 0]], theta=500000.0)
    o, lse = gpu_run(w, x, split_tiles=split, rope=rope)
    compare(w, x, o, lse, rope=rope)


@pytest.mark.parametrize("case", [
    (5, 3000, 64, 8, 128, 64, (0, 512, 512, 512, 512, 512, 512, 512), 0, 0, 16),
    (3, (1, 63, 650), 16, 4, 64, 16, (0, 1, 7, 64), 1, 16, 4),
    (2, 4097, 32, 4, 128, 32, (4096, 0, 100, 1), 0, 64, None),
])
def test_decode_relocated_matches_oracle(case):
    n, kv, hq, hkv, d, p, windows, style, dims, pps = case
    kvs = (kv,) * n if isinstance(kv, int) else tuple(kv)
    w = wl.Workload("rope_dec", kvs, (1,) * len(kvs), hq, hkv, d, p, tuple(windows), seed=n + d, decode=True)
    x = wl.make_inputs(w)
    rng = np.random.default_rng(n)
    deltas = rng.integers(-5000, 200000, size=(len(kvs), hkv)).tolist()
    deltas[0][0] = 0
    rope = dict(deltas=deltas, style=style, dims=dims)
    o, lse = gpu_run(w, x, mode="decode", pps=pps, rope=rope)
    compare(w, x, o, lse, rope=rope)


def test_zero_or_cleared_offsets_are_bitwise_the_plain_path():
    import torch
    from long_context_serving_amd import runner as R
    w = wl.small_workload("rope_zero", (500,), (500,), 8, 2, 128, 64, (0, 100), seed=4)
    x = wl.make_inputs(w)
    o0, l0 = gpu_run(w, x)
    o1, l1 = gpu_run(w, x, rope=dict(deltas=[[0, 0]]))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    run = R.WorkloadRun(w, R.to_device(w, x), deltas=[[900, 900]])
    if PREFILL_KERNEL:
        run.ctx.set_tuning(S.TUNE_PREFILL_KERNEL, PREFILL_KERNEL)
    run.load()
    run.ctx.set_relocation(0, None)
    o2, l2 = run.prefill()
    torch.cuda.synchronize()
    assert np.array_equal(o0, S.bf16_bits(o2)) and np.array_equal(l0, l2.cpu().numpy().astype(np.float64))
    run.close()


def test_relocated_decode_matches_relocated_prefill_of_last_token():
    w = wl.Workload("rope_dvp", (700, 1200, 64), (1, 1, 1), 16, 4, 128, 64, (0, 100, 300, 5), seed=3, decode=True)
    x = wl.make_inputs(w)
    rope = dict(deltas=[[10, 20, 30, 40], [0, 7000, 0, 7000], [123, 0, 0, 1]], style=1)
    od, ld = gpu_run(w, x, mode="decode", rope=rope)
    op, lp = gpu_run(w, x, mode="prefill", rope=rope)
    compare(w, x, od, ld, rope=rope)
    compare(w, x, op, lp, rope=rope)


@pytest.mark.parametrize("style,dims", [(0, 0), (1, 64)])
def test_canonical_cache_with_relocation_reproduces_true_position_cache(style, dims):
    """A document of n tokens sits at offset delta of a request.  Cache A holds
    its keys encoded at their true positions delta + t; cache B holds the keys
    encoded at canonical positions t and relocates the queries by delta.  Both
    match their oracle, and the two oracles agree up to bf16 rounding."""
    n, delta, theta = 600, 20000, 10000.0
    w = wl.small_workload("rope_doc", (n,), (n,), 16, 4, 128, 64, (0, 64, 200, 600), seed=21 + style)
    x = wl.make_inputs(w)
    rng = np.random.default_rng(77)
    raw_q = rng.standard_normal((n, 16, 128), dtype=np.float32)
    raw_k = rng.standard_normal((n, 4, 128), dtype=np.float32)
    pos = np.arange(n)
    enc = lambda a, p: wl.to_bf16_bits(RP.rope_rotate(a, p[:, None], theta, style, dims).astype(np.float32))
    q_abs = enc(raw_q, delta + pos)
    xa = dataclasses.replace(x, q=q_abs, k=enc(raw_k, delta + pos))
    xb = dataclasses.replace(x, q=q_abs, k=enc(raw_k, pos))
    oa, la = gpu_run(w, xa)
    compare(w, xa, oa, la)
    rope = dict(deltas=[[delta] * 4], style=style, dims=dims)
    ob, lb = gpu_run(w, xb, rope=rope)
    compare(w, xb, ob, lb, rope=rope)
    # the caches differ only by bf16 rounding of keys and relocated queries
    do = np.abs(A.bf16_bits_to_f64(oa) - A.bf16_bits_to_f64(ob)).max()
    dl = np.abs(la - lb).max()
    say(f"  true-position cache vs relocated canonical cache: max|do|={do:.3e} max|dlse|={dl:.3e}")
    assert do < 5e-2 and dl < 5e-2
