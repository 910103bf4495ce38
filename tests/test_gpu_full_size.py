"""GPU parity at the named workloads' full sizes, in the launch
configuration the benchmark times.  The oracle computes a sample of rows
one by one: every boundary row (first and last queries of each sequence and
chunk, window and page edges) plus seeded random rows."""

import numpy as np
import pytest

from long_context_serving_amd import segkv as S
from long_context_serving_amd import workloads as wl

from gpu_helpers import compare, gpu_run, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load_library()


@pytest.mark.parametrize("name", ["mistral7b_prefill_L8192", "llama70b_varlen_prefill", "chunked_prefill_128k"])
def test_full_size_prefill(name):
    w = wl.WORKLOADS[name]
    x = wl.make_inputs(w)
    o, lse = gpu_run(w, x)
    rows = [sample_rows(w, b, n_random=96 if w.n_seqs > 1 else 256) for b in range(w.n_seqs)]
    compare(w, x, o, lse, rows_per_seq=rows)


def test_full_size_decode():
    w = wl.DECODE_32K
    x = wl.make_inputs(w)
    o, lse = gpu_run(w, x, mode="decode")
    compare(w, x, o, lse)


@pytest.mark.parametrize("name", ["mistral7b_prefill_L8192", "llama70b_varlen_prefill", "chunked_prefill_128k"])
def test_full_size_all_global_arms_sampled(name):
    """The comparison arm the benchmark times beside each prefill workload:
    the same inputs and kernels with every head global."""
    w = wl.WORKLOADS[name]
    x = wl.make_inputs(w)
    g = (0,) * w.num_kv_heads
    o, lse = gpu_run(w, x, windows=g)
    rows = [sample_rows(w, b, n_random=48 if w.n_seqs > 1 else 96) for b in range(w.n_seqs)]
    compare(w, x, o, lse, rows_per_seq=rows, windows=g)


def _local_deltas(w, offset):
    return [[offset if win > 0 else 0 for win in w.windows] for _ in range(w.n_seqs)]


def test_full_size_relocated_headline_prefill():
    """The relocation arm: every local head of the Llama-3.3-70B-shaped varlen
    prefill relocated by a document offset of 8192 (global heads by 0)."""
    w = wl.LLAMA70B_VARLEN_PREFILL
    x = wl.make_inputs(w)
    rope = dict(deltas=_local_deltas(w, 8192))
    o, lse = gpu_run(w, x, rope=rope)
    rows = [sample_rows(w, b, n_random=48) for b in range(w.n_seqs)]
    compare(w, x, o, lse, rows_per_seq=rows, rope=rope)


def test_full_size_relocated_decode():
    w = wl.DECODE_32K
    x = wl.make_inputs(w)
    rope = dict(deltas=_local_deltas(w, 8192))
    o, lse = gpu_run(w, x, mode="decode", rope=rope)
    compare(w, x, o, lse, rope=rope)


def test_full_size_decode_over_31_forks():
    """The fork arm: 31 sequences forked from one parent of 32767 tokens, each
    appending its own query token, decoded together; every (fork, head) row
    against the oracle on that fork's own history."""
    import torch
    from oracle import attention as A
    from gpu_helpers import O_TOL, LSE_TOL, say
    dw = wl.DECODE_32K
    n, L = dw.n_seqs, dw.kv_lens[0]
    fw = wl.Workload("fork_parent", (L - 1 + n,), (n,), dw.num_q_heads, dw.num_kv_heads, dw.head_dim,
                     dw.page_size, dw.windows, seed=dw.seed + 50)
    x = wl.make_inputs(fw)
    k, v, q = S.bf16_tensor(x.k), S.bf16_tensor(x.v), S.bf16_tensor(x.q)
    say(f"fork decode: {n} forks of a {L - 1}-token parent")
    ctx = S.SegKV(1, dw.num_q_heads, dw.num_kv_heads, dw.head_dim, dw.page_size, n + 1, n * 1000,
                  list(dw.windows), softmax_scale=dw.scale, page_order_seed=dw.page_order_seed)
    ctx.append_pages(0, [n], [L - 1], [0], k[: L - 1].contiguous(), v[: L - 1].contiguous())
    for i in range(n):
        ctx.fork(n, i)
    ctx.append_pages(0, list(range(n)), [1] * n, [1] * n, k[L - 1:].contiguous(), v[L - 1:].contiguous())
    o, lse = ctx.decode(0, list(range(n)), q)
    torch.cuda.synchronize()
    ob = A.bf16_bits_to_f64(S.bf16_bits(o))
    lg = lse.cpu().numpy().astype(np.float64)
    ctx.close()
    kf = A.bf16_bits_to_f64(x.k)
    vf = A.bf16_bits_to_f64(x.v)
    qf = A.bf16_bits_to_f64(x.q)
    worst_o = worst_l = 0.0
    for i in range(n):
        hist = np.concatenate([np.arange(L - 1), [L - 1 + i]])
        ro, rl = A.attend_sequence(qf[i:i + 1], kf[hist], vf[hist], dw.windows, dw.scale)
        worst_o = max(worst_o, float(np.abs(ob[i] - ro[0]).max()))
        worst_l = max(worst_l, float(np.abs(lg[i] - rl[0]).max()))
    say(f"  max|do|={worst_o:.3e} max|dlse|={worst_l:.3e}")
    assert worst_o <= O_TOL and worst_l <= LSE_TOL
