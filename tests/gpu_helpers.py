"""Shared helpers of the GPU parity tests: run a workload through libsegkv
and compare with the fp64 oracle on the same seeded inputs."""

from __future__ import annotations

import os
import sys

import numpy as np

from long_context_serving_amd import runner as R
from long_context_serving_amd import segkv as S
from long_context_serving_amd import workloads as wl
from oracle import attention as A
from oracle import rope as RP

O_TOL = 2e-2    # max-abs on bf16 outputs against the unrounded fp64 oracle
LSE_TOL = 1e-3  # max-abs on fp32 log-sum-exp

# Prefill kernel the parity runs select (SEGKV_TUNE_PREFILL_KERNEL): the
# suite can be run once per kernel variant.
PREFILL_KERNEL = int(os.environ.get("SEGKV_TEST_PREFILL_KERNEL", "0"))


def say(*msg):
    print("[gpu]", *msg, file=sys.stderr, flush=True)


CANARY_BITS = 0x7F7F  # bf16 bit pattern of every byte pair the library must not write (3.39e38)
GUARD_PAGES = 4


class GuardedPools:
    """K and V pools with canary guard pages on both sides: the whole
    allocation is filled with a pattern before the context is created; after
    a run, the guard pages and every page no segment ever held must still
    hold it.  A scatter or copy-on-write write to a wrong page id, or past
    either end of the pool, shows up here even when no later read meets it."""

    def __init__(self, num_pages, page_size, head_dim, device="cuda"):
        import torch
        self.n, self.g = int(num_pages), GUARD_PAGES
        shape = (self.n + 2 * self.g, page_size, head_dim)
        self.k_all = torch.empty(shape, dtype=torch.bfloat16, device=device)
        self.v_all = torch.empty((self.n + 2 * self.g, head_dim, page_size), dtype=torch.bfloat16, device=device)
        for t in (self.k_all, self.v_all):
            t.view(torch.int16).fill_(CANARY_BITS)
        self.k = self.k_all[self.g:self.g + self.n]
        self.v = self.v_all[self.g:self.g + self.n]
        self.used = set()

    @property
    def pools(self):
        return self.k, self.v

    def note(self, ctx):
        """Record every page some segment of ctx holds now."""
        for layer in range(ctx.num_layers):
            for s in range(ctx.max_seqs):
                for g in range(ctx.num_kv_heads):
                    self.used.update(int(p) for p in ctx.page_table(layer, s, g)[2])

    def check(self):
        import torch
        if self.k_all.is_cuda:
            torch.cuda.synchronize()
        for name, t in (("K", self.k_all), ("V", self.v_all)):
            intact = (t.view(torch.int16) == CANARY_BITS).flatten(1).all(dim=1).cpu().numpy()
            assert intact[:self.g].all(), f"{name} guard pages before the pool were written"
            assert intact[self.g + self.n:].all(), f"{name} guard pages after the pool were written"
            never = np.array(sorted(set(range(self.n)) - self.used), dtype=np.int64)
            if len(never):
                bad = never[~intact[self.g + never]]
                assert len(bad) == 0, f"{name} pages {bad[:8].tolist()} were written but never held by a segment"
        return True


def gpu_run(w, x, mode="prefill", seed=None, windows=None, split_tiles=None, pps=None, repeat=1, rope=None,
            prefill_kernel=None):
    """``rope``: dict(deltas=[n_seqs][Hkv], theta=, style=, dims=) for query
    relocation, or None.  ``prefill_kernel``: SEGKV_TUNE_PREFILL_KERNEL value
    (None = PREFILL_KERNEL)."""
    import torch
    say(f"{mode} {w.name} kv={w.kv_lens[:4]} q={w.q_lens[:4]} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"D={w.head_dim} P={w.page_size} W={windows or w.windows} seed={seed} split={split_tiles} pps={pps}"
        f" kernel={PREFILL_KERNEL if prefill_kernel is None else prefill_kernel}"
        + ("" if rope is None else f" rope={rope}"))
    dev = R.to_device(w, x)
    rkw = {} if rope is None else dict(deltas=rope["deltas"], rope_theta=rope.get("theta", 0.0),
                                       rope_style=rope.get("style", 0), rope_dims=rope.get("dims", 0))
    canary = GuardedPools(R.pages_for(w), w.page_size, w.head_dim)
    run = R.WorkloadRun(w, dev, page_order_seed=seed, windows=windows, pools=canary.pools, **rkw)
    try:
        kernel = PREFILL_KERNEL if prefill_kernel is None else prefill_kernel
        if kernel:
            run.ctx.set_tuning(S.TUNE_PREFILL_KERNEL, kernel)
        if split_tiles is not None:
            run.ctx.set_tuning(S.TUNE_PREFILL_SPLIT_TILES, split_tiles)
        if pps is not None:
            run.ctx.set_tuning(S.TUNE_DECODE_MIN_PAGES, pps)
        run.load(after_append=canary.note)
        outs = []
        for _ in range(repeat):
            o, lse = run.prefill() if mode == "prefill" else run.decode()
            torch.cuda.synchronize()
            outs.append((S.bf16_bits(o), lse.cpu().numpy().astype(np.float64)))
        canary.check()
        return outs if repeat > 1 else outs[0]
    finally:
        run.close()


def compare(w, x, o_bits, lse, rows_per_seq=None, windows=None, o_tol=O_TOL, lse_tol=LSE_TOL, rope=None):
    """Oracle rows vs GPU rows; returns (max |do|, max |dlse|)."""
    if rope is None:
        ref = A.attend_batch(x.q, x.k, x.v, x.cu_q, x.cu_kv, windows or w.windows, w.scale, rows_per_seq)
    else:
        ref = RP.attend_batch_relocated(x.q, x.k, x.v, x.cu_q, x.cu_kv, windows or w.windows, w.scale,
                                        rope["deltas"], rope.get("theta") or 10000.0, rope.get("style", 0),
                                        rope.get("dims", 0), rows_per_seq)
    worst_o = worst_l = 0.0
    for b, (ro, rl) in enumerate(ref):
        rows = np.arange(w.q_lens[b]) if rows_per_seq is None else np.asarray(rows_per_seq[b])
        if len(rows) == 0:
            continue
        go = A.bf16_bits_to_f64(o_bits[x.cu_q[b] + rows])
        gl = lse[x.cu_q[b] + rows]
        assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
        worst_o = max(worst_o, float(np.max(np.abs(go - ro))))
        worst_l = max(worst_l, float(np.max(np.abs(gl - rl))))
    say(f"  max|do|={worst_o:.3e} max|dlse|={worst_l:.3e}")
    assert worst_o <= o_tol, worst_o
    assert worst_l <= lse_tol, worst_l
    return worst_o, worst_l


def sample_rows(w, b, n_random=512, seed=0):
    """Boundary rows (first/last of the chunk, window and page edges) plus
    seeded random rows of sequence b."""
    q_len, kv_len = w.q_lens[b], w.kv_lens[b]
    base = kv_len - q_len
    rows = {0, 1, q_len - 1, q_len - 2}
    edges = set()
    for wdw in set(w.windows) - {0}:
        for p in (wdw - 2, wdw - 1, wdw, wdw + 1, base + wdw - 1, base + wdw):
            edges.add(p)
    for k in range(1, 5):
        edges.update({k * w.page_size - 1, k * w.page_size, 64 * k - 1, 64 * k})
    for p in edges:
        t = p - base
        if 0 <= t < q_len:
            rows.add(t)
    rng = np.random.default_rng(seed + b)
    rows.update(int(t) for t in rng.integers(0, q_len, size=min(n_random, q_len)))
    return np.array(sorted(r for r in rows if 0 <= r < q_len), dtype=np.int64)
