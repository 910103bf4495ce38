#!/usr/bin/env python3
"""Benchmark of segmented paged attention on one MI355X.

One step = one pass of the attention hot path over one batch of the
workload: release the batch's sequences, append their cache fill (no
queries) and their query tokens (page allocation, table upload, KV
scatter), then run varlen prefill (and the combine of split rows).  Inputs
are resident in HBM before the timed region.

Headline: the Llama-3.3-70B-shaped varlen layer prefill, the largest
workload that fits one GPU (4 sequences of [29127, 12589, 8841, 23919]
tokens, 64 query / 8 KV heads, D = 128, 1 global + 7 local KV heads with
W = 2048, page 64, random page order).  value = visible-token TFLOP/s = 4 *
D * (visible (query head, query, key) pairs) per step / step time.

In the same JSON line:
  roofline      the prefill's kernel rate: visible FLOPs over the prefill
                launch plus its combine launch, both timed by HIP events that
                the library records around each launch on its stream, against
                the 2.5 PFLOP/s dense bf16 MFMA peak (traffic: rocprofv3
                counter bytes when they were taken on the current kernel
                source, else null);
  all_global    the same steps with every head forced global;
  protocol      3 unmeasured + 10 measured (segmented, all-global) pairs,
                p50 / p95 of prefill + combine kernel time;
  workloads     the 128K chunked prefill (122880 cached + 8192 queries) and
                the Mistral-7B-shaped L = 8192 prefill, each with the same
                fields;
  relocation    query-side RoPE relocation: the headline prefill and the
                decode with every local head's queries relocated by a
                document offset (global heads at offset 0), and the cost over
                the plain kernels;
  decode        visible-KV GB/s of split-KV decode + combine at 32K x 31
                sequences against 8 TB/s, its all-global arm and the oracle's
                rate on the host;
  router        attention-mass token scores of the Mistral-7B-shaped prefill
                (a second MFMA pass over the visible pairs, QK only: 2 D FLOPs
                per pair) and the top-k (k = L/4) that routes tokens to the
                dense FFN;
  merge         the head-decomposition merge of a reused 128K-token document:
                algorithmic GB/s against 8 TB/s;
  fork          copy-on-write forks: the 32K x 31 decode with the 31 sequences
                forked from one 32767-token parent: pages in use against 31
                unshared copies, and the decode kernel over the forks;
  cpu_baseline  the fp64 oracle on a bounded sample of the headline workload.

Warm-up: each arm first runs its own step until 0.25 s of wall time has
passed (the GPU's clock settles under sustained load and drops back when it
idles), then the W warm-up steps, then the K timed steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "visible-token attention TFLOP/s (prefill) & visible-KV GB/s (decode), 1 MI355X"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "long_context_serving_amd", "csrc")
# Sources whose digest identifies each measured kernel: its own file plus the
# shared device helpers and the argument layouts.
KERNEL_SRC = {
    "prefill": ["prefill.hip", "kernels_common.h", "page_layout.h", "segkv_internal.h"],
    "score": ["score.hip", "kernels_common.h", "page_layout.h", "segkv_internal.h"],
    "decode": ["decode.hip", "kernels_common.h", "page_layout.h", "segkv_internal.h"],
    "merge": ["merge.hip", "kernels_common.h", "segkv_internal.h"],
}
RELOCATION_OFFSET = 8192    # document offset of the relocation arm


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash(kind: str) -> str:
    """First 16 hex digits of the sha256 over the kernel's source files."""
    h = hashlib.sha256()
    for name in KERNEL_SRC[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    ("<kind>_<workload>"), or None when the kernel's sources changed since
    the counters were taken (or a prefill variant other than the default is
    timed)."""
    kind = key.split("_", 1)[0]
    if kind not in KERNEL_SRC or (kind == "prefill" and PREFILL_KERNEL not in (0, 1)):
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(key)
    if not e or e.get("kernel_source_sha256_16") != kernel_source_hash(kind):
        return None
    return e.get("bytes_per_launch")


def sync():
    import torch
    torch.cuda.synchronize()


def pct(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q)) if xs else None


def kernel_avg(ctx, kernel):
    ms, n = ctx.read_timing(kernel)
    return (ms / n if n else 0.0), n


# --------------------------------------------------------------- prefill

WARM_CLOCK_S = 0.25


def warm_clock(step):
    """Run ``step`` until WARM_CLOCK_S of wall time has passed (untimed)."""
    t0 = time.perf_counter()
    while True:
        step()
        sync()
        if time.perf_counter() - t0 >= WARM_CLOCK_S:
            return


PREFILL_KERNEL = 0  # SEGKV_TUNE_PREFILL_KERNEL of every prefill arm (--prefill-kernel)


def prefill_arm(w, dev, steps, warmup, windows=None, split_tiles=None, deltas=None):
    import torch
    from long_context_serving_amd import runner as R
    from long_context_serving_amd import segkv as S
    run = R.WorkloadRun(w, dev, windows=windows, deltas=deltas)
    if split_tiles:
        run.ctx.set_tuning(S.TUNE_PREFILL_SPLIT_TILES, split_tiles)
    if PREFILL_KERNEL:
        run.ctx.set_tuning(S.TUNE_PREFILL_KERNEL, PREFILL_KERNEL)
    o = torch.empty_like(dev.q)
    lse = torch.empty(dev.q.shape[:2], dtype=torch.float32, device=dev.q.device)

    def step():
        run.reset()
        run.load()
        run.prefill(o, lse)

    warm_clock(step)
    for _ in range(warmup):
        step()
    sync()
    # The step time comes from a loop without timing events (events add a
    # few microseconds at every kernel boundary); the kernel times come from
    # the same number of steps run next with events around the prefill and
    # combine launches, and the append's scatter is timed after that.
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    sync()
    dt = (time.perf_counter() - t0) / steps
    run.ctx.set_timing(True, [S.KERNEL_PREFILL, S.KERNEL_COMBINE])
    for _ in range(steps):
        step()
    sync()
    k_ms, k_n = kernel_avg(run.ctx, S.KERNEL_PREFILL)
    c_ms, c_n = kernel_avg(run.ctx, S.KERNEL_COMBINE)
    run.ctx.set_timing(True, [S.KERNEL_SCATTER])
    n_sc = max(2, steps // 4)
    for _ in range(n_sc):
        step()
    sync()
    s_ms, s_n = kernel_avg(run.ctx, S.KERNEL_SCATTER)
    run.ctx.set_timing(False)
    # combine time per step (a step has a combine launch only when rows are split)
    c_step = c_ms * c_n / max(k_n, 1)
    return run, {"ms_per_step": dt * 1e3, "prefill_kernel_ms": k_ms, "prefill_launches": k_n,
                 "combine_kernel_ms": c_step, "scatter_kernel_ms_per_launch": s_ms,
                 "scatter_launches_per_step": s_n / n_sc}


def paired_protocol(run_a, run_b, warm=3, measured=10):
    """The pages' timing protocol at kernel level: unmeasured warm pairs, then
    measured (segmented, all-global) pairs; returns per-arm prefill +
    combine kernel times."""
    from long_context_serving_amd import segkv as S
    times = {"segmented": [], "all_global": []}
    for i in range(warm + measured):
        for name, run in (("segmented", run_a), ("all_global", run_b)):
            run.reset()
            run.load()
            run.ctx.set_timing(True)
            run.prefill()
            ms, _ = run.ctx.read_timing(S.KERNEL_PREFILL)
            cms, _ = run.ctx.read_timing(S.KERNEL_COMBINE)
            run.ctx.set_timing(False)
            if i >= warm:
                times[name].append(ms + cms)
    return {k: {"p50_ms": pct(v, 50), "p95_ms": pct(v, 95)} for k, v in times.items()}


def prefill_report(w, dev, steps, warmup, with_global=True, with_protocol=True):
    """Segmented arm (kept open for later arms) and its report: step rate,
    kernel roofline over prefill + combine, the all-global arm and the
    paired protocol."""
    from long_context_serving_amd import metrics as M
    flops = M.prefill_flops(w)
    g = (0,) * w.num_kv_heads
    flops_g = M.prefill_flops(w, windows=g)
    log(f"prefill {w.name} segmented")
    run, seg = prefill_arm(w, dev, steps, warmup)
    log(f"  {seg}")
    kern = seg["prefill_kernel_ms"] + seg["combine_kernel_ms"]
    achieved = flops / (kern * 1e-3) / 1e12
    rep = {
        "workload": w.name, "value": flops / (seg["ms_per_step"] * 1e-3) / 1e12, "unit": "TFLOP/s",
        "visible_flops": flops, "ms_per_step": seg["ms_per_step"],
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic("prefill_" + w.name),
                     "kernel": f"prefill_kernel<{w.head_dim},{w.page_size}> + combine_kernel<{w.head_dim}>",
                     "avg_launch_ms": seg["prefill_kernel_ms"], "combine_ms_per_step": seg["combine_kernel_ms"],
                     "prefill_launch_only_tflops": flops / (seg["prefill_kernel_ms"] * 1e-3) / 1e12},
        "step_breakdown": seg,
    }
    if with_global:
        log(f"prefill {w.name} all-global")
        run_g, glob = prefill_arm(w, dev, steps, warmup, windows=g)
        log(f"  {glob}")
        kern_g = glob["prefill_kernel_ms"] + glob["combine_kernel_ms"]
        rep["all_global"] = {
            "value": flops_g / (glob["ms_per_step"] * 1e-3) / 1e12, "unit": "TFLOP/s", "visible_flops": flops_g,
            "ms_per_step": glob["ms_per_step"], "prefill_kernel_ms": glob["prefill_kernel_ms"],
            "combine_kernel_ms": glob["combine_kernel_ms"], "kernel_tflops": flops_g / (kern_g * 1e-3) / 1e12,
            "kernel_frac": flops_g / (kern_g * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "segmented_speedup_step": glob["ms_per_step"] / seg["ms_per_step"],
            "segmented_speedup_kernel": kern_g / kern}
        if with_protocol:
            rep["protocol"] = paired_protocol(run, run_g)
        run_g.close()
    return run, rep


# ---------------------------------------------------------------- decode

def decode_arm(w, dev, steps, warmup, windows=None, deltas=None):
    import torch
    from long_context_serving_amd import runner as R
    from long_context_serving_amd import segkv as S
    run = R.WorkloadRun(w, dev, windows=windows, deltas=deltas).load()
    o = torch.empty_like(dev.q)
    lse = torch.empty(dev.q.shape[:2], dtype=torch.float32, device=dev.q.device)
    warm_clock(lambda: run.decode(o, lse))
    for _ in range(warmup):
        run.decode(o, lse)
    sync()
    # Step time without timing events, then kernel times over as many steps.
    t0 = time.perf_counter()
    for _ in range(steps):
        run.decode(o, lse)
    sync()
    dt = (time.perf_counter() - t0) / steps
    run.ctx.set_timing(True)
    for _ in range(steps):
        run.decode(o, lse)
    sync()
    d_ms, d_n = kernel_avg(run.ctx, S.KERNEL_DECODE_SPLIT)
    c_ms, _ = kernel_avg(run.ctx, S.KERNEL_COMBINE)
    run.ctx.set_timing(False)
    pages = run.ctx.num_pages - run.ctx.free_pages()
    run.close()
    return {"ms_per_step": dt * 1e3, "split_kernel_ms": d_ms, "combine_kernel_ms": c_ms, "launches": d_n,
            "pages_in_use": pages}


# ----------------------------------------------------------- cpu baseline

def router_arm(w, dev, steps, warmup, flops_qk):
    import torch
    from long_context_serving_amd import runner as R
    from long_context_serving_amd import segkv as S
    run = R.WorkloadRun(w, dev).load()
    o, lse = run.prefill()
    scores = torch.empty(dev.q.shape[0], dtype=torch.float32, device=dev.q.device)
    k = [n // 4 for n in w.q_lens]
    idx = torch.empty(sum(k), dtype=torch.int32, device=dev.q.device)

    def call():
        run.ctx.token_scores(0, run.seq_ids, w.q_lens, dev.q, lse, scores)
        run.ctx.topk(w.q_lens, scores, k, idx)

    warm_clock(call)
    for _ in range(warmup):
        call()
    sync()
    # Call time without timing events, then kernel times over as many calls.
    t0 = time.perf_counter()
    for _ in range(steps):
        run.ctx.token_scores(0, run.seq_ids, w.q_lens, dev.q, lse, scores)
        run.ctx.topk(w.q_lens, scores, k, idx)
    sync()
    dt = (time.perf_counter() - t0) / steps
    run.ctx.set_timing(True, [S.KERNEL_SCORE, S.KERNEL_SCORE_REDUCE, S.KERNEL_TOPK])
    for _ in range(steps):
        run.ctx.token_scores(0, run.seq_ids, w.q_lens, dev.q, lse, scores)
        run.ctx.topk(w.q_lens, scores, k, idx)
    sync()
    s_ms, _ = kernel_avg(run.ctx, S.KERNEL_SCORE)
    r_ms, _ = kernel_avg(run.ctx, S.KERNEL_SCORE_REDUCE)
    k_ms, _ = kernel_avg(run.ctx, S.KERNEL_TOPK)
    run.ctx.set_timing(False)
    run.close()
    tf = flops_qk / (s_ms * 1e-3) / 1e12
    return {"workload": w.name, "k_per_seq": k, "ms_per_call": dt * 1e3, "score_kernel_ms": s_ms,
            "reduce_kernel_ms": r_ms, "topk_kernel_ms": k_ms, "qk_flops": flops_qk,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic("score_" + w.name),
                         "kernel": "score_kernel<128,64>",
                         "avg_launch_ms": s_ms}}


def merge_arm(mw, steps, warmup):
    import torch
    from long_context_serving_amd import metrics as M
    from long_context_serving_amd import segkv as S
    from long_context_serving_amd import workloads as wl
    torch.cuda.empty_cache()  # fresh allocations for the multi-GB buffers, whatever ran before
    mi = wl.make_merge_inputs(mw)
    by = M.merge_bytes(mi.mode, mw.head_dim)
    ctx = S.SegKV(1, mw.num_q_heads, mw.num_kv_heads, mw.head_dim, 64, 1, 4, [0] * mw.num_kv_heads)
    args = (S.bf16_tensor(mi.o_a), torch.from_numpy(mi.lse_a).cuda(), S.bf16_tensor(mi.o_b),
            torch.from_numpy(mi.lse_b).cuda(), torch.from_numpy(mi.mode).cuda())
    del mi
    o = torch.empty_like(args[0])
    lse = torch.empty_like(args[1])
    warm_clock(lambda: ctx.merge(*args, o=o, lse=lse))
    for _ in range(warmup):
        ctx.merge(*args, o=o, lse=lse)
    sync()
    # Call time without timing events, then kernel times over as many calls.
    t0 = time.perf_counter()
    for _ in range(steps):
        ctx.merge(*args, o=o, lse=lse)
    sync()
    dt = (time.perf_counter() - t0) / steps
    ctx.set_timing(True, [S.KERNEL_MERGE])
    for _ in range(steps):
        ctx.merge(*args, o=o, lse=lse)
    sync()
    k_ms, k_n = kernel_avg(ctx, S.KERNEL_MERGE)
    ctx.set_timing(False)
    ctx.close()
    gbs = by["total"] / (k_ms * 1e-3) / 1e9
    return {"workload": mw.name, "rows": mw.rows, "num_q_heads": mw.num_q_heads, "head_dim": mw.head_dim,
            "value": gbs, "unit": "GB/s", "bytes": by, "ms_per_call": dt * 1e3, "kernel_ms": k_ms,
            "launches": k_n,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": measured_traffic("merge_" + mw.name),
                         "kernel": "merge_kernel<128>", "avg_launch_ms": k_ms}}


def fork_arm(dw, steps, warmup, pages_unshared):
    """31 forks of one parent of kv_len - 1 tokens, each appending one query."""
    import torch
    from long_context_serving_amd import metrics as M
    from long_context_serving_amd import segkv as S
    from long_context_serving_amd import workloads as wl
    n, L = dw.n_seqs, dw.kv_lens[0]
    torch.cuda.empty_cache()
    fw = wl.Workload("fork_parent", (L - 1 + n,), (n,), dw.num_q_heads, dw.num_kv_heads, dw.head_dim,
                     dw.page_size, dw.windows, seed=dw.seed + 50)
    x = wl.make_inputs(fw)
    k, v, q = S.bf16_tensor(x.k), S.bf16_tensor(x.v), S.bf16_tensor(x.q)
    del x
    ctx = S.SegKV(1, dw.num_q_heads, dw.num_kv_heads, dw.head_dim, dw.page_size, n + 1, pages_unshared,
                  list(dw.windows), softmax_scale=dw.scale, page_order_seed=dw.page_order_seed)
    parent = n
    ctx.append_pages(0, [parent], [L - 1], [0], k[: L - 1].contiguous(), v[: L - 1].contiguous())
    parent_pages = ctx.num_pages - ctx.free_pages()
    t0 = time.perf_counter()
    for i in range(n):
        ctx.fork(parent, i)
    fork_us = (time.perf_counter() - t0) / n * 1e6
    ctx.append_pages(0, list(range(n)), [1] * n, [1] * n, k[L - 1:].contiguous(), v[L - 1:].contiguous())
    used = ctx.num_pages - ctx.free_pages()
    per_fork = (used - parent_pages) / n
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    ids = list(range(n))
    warm_clock(lambda: ctx.decode(0, ids, q, o, lse))
    for _ in range(warmup):
        ctx.decode(0, ids, q, o, lse)
    sync()
    ctx.set_timing(True, [S.KERNEL_DECODE_SPLIT, S.KERNEL_COMBINE])
    for _ in range(steps):
        ctx.decode(0, ids, q, o, lse)
    sync()
    d_ms, _ = kernel_avg(ctx, S.KERNEL_DECODE_SPLIT)
    c_ms, _ = kernel_avg(ctx, S.KERNEL_COMBINE)
    ctx.set_timing(False)
    ctx.close()
    by = M.decode_bytes(dw)
    return {"workload": "decode_32k_x31 as 31 forks of one parent", "pages_in_use": used,
            "pages_parent": parent_pages, "pages_per_fork": per_fork, "pages_unshared": pages_unshared,
            "page_ratio": pages_unshared / used, "forks_fitting_in_unshared_pool":
                int((pages_unshared - parent_pages) // per_fork) if per_fork else None,
            "fork_call_us": fork_us, "split_kernel_ms": d_ms, "combine_kernel_ms": c_ms,
            "visible_kv_gbs": by["total"] / ((d_ms + c_ms) * 1e-3) / 1e9,
            "note": "forks read the shared pages, so part of the visible bytes come from cache"}


def local_head_deltas(w, offset):
    """Every local KV head of every sequence relocated by ``offset``; global
    heads (recomputed online at their true positions) by 0."""
    return [[offset if win > 0 else 0 for win in w.windows] for _ in range(w.n_seqs)]


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        return None


def cpu_baseline(w, x, budget_s=30.0):
    """The fp64 oracle, as it stands, on a seeded sample of query rows of the
    workload (all heads; rows spread over the sequences in proportion to
    their query counts), timed on the host cores."""
    from oracle import attention as A
    from long_context_serving_amd import metrics as M
    threads = _blas_threads()
    rng = np.random.default_rng(2024)
    q_tot = sum(w.q_lens)

    def run(n):
        rows = []
        for b, ql in enumerate(w.q_lens):
            nb = max(1, int(round(n * ql / q_tot))) if ql else 0
            rows.append(np.sort(rng.choice(ql, size=min(nb, ql), replace=False)) if nb else np.zeros(0, np.int64))
        t0 = time.perf_counter()
        A.attend_batch(x.q, x.k, x.v, x.cu_q, x.cu_kv, w.windows, w.scale, rows_per_seq=rows)
        dt = time.perf_counter() - t0
        return dt, sum(M.prefill_flops_rows(w, b, r) for b, r in enumerate(rows)), sum(len(r) for r in rows)

    n = 64
    t, flops, n = run(n)
    while t < budget_s / 3 and n < q_tot:   # grow the sample until it is ~budget_s/3 of work
        n = int(min(q_tot, n * max(2.0, min(8.0, budget_s / 3 / max(t, 1e-3)))))
        t, flops, n = run(n)
    reps = 1
    if t < budget_s / 3:                     # the whole workload is cheap: repeat it
        reps = int(np.ceil(budget_s / 3 / t))
        t0 = time.perf_counter()
        for _ in range(reps):
            _, flops, n = run(n)
        t = (time.perf_counter() - t0) / reps
    out = {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads or os.cpu_count(),
           "kind": "oracle",
           "sample": f"{n} of {q_tot} query rows (seeded, spread over the {w.n_seqs} sequences), all "
                     f"{w.num_q_heads} query heads, of {w.name}; {t:.1f} s per pass, {reps} pass(es); fp64 "
                     f"numpy, BLAS threads={threads}, host cpus={os.cpu_count()}"}
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        return out
    with threadpool_limits(limits=1):
        n1 = 8
        t1, f1, n1 = run(n1)
        while t1 < budget_s / 9 and n1 < q_tot:
            n1 = int(min(q_tot, n1 * max(2.0, min(8.0, budget_s / 9 / max(t1, 1e-3)))))
            t1, f1, n1 = run(n1)
    out["single_thread"] = {"value": f1 / t1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                            "sample": f"{n1} of {q_tot} query rows (seeded), {t1:.1f} s"}
    return out


def cpu_baseline_decode(w, x, budget_s=20.0):
    """The fp64 oracle on the decode workload's sequences (one query row each,
    all heads), as visible-KV GB/s: the same algorithmic bytes as the GPU
    figure, over the oracle's wall time, on a growing prefix of the batch."""
    from oracle import attention as A
    from long_context_serving_amd import metrics as M
    threads = _blas_threads()
    by = M.decode_bytes(w)["total"] / w.n_seqs

    def run(n):
        t0 = time.perf_counter()
        cu_q = x.cu_q[:n + 1]
        cu_kv = x.cu_kv[:n + 1]
        A.attend_batch(x.q, x.k, x.v, cu_q, cu_kv, w.windows, w.scale)
        return time.perf_counter() - t0

    n = 1
    t = run(n)
    while t < budget_s / 2 and n < w.n_seqs:
        n = min(w.n_seqs, n * 2)
        t = run(n)
    reps = 1
    if t < budget_s / 2:  # the whole batch is cheap: time repeated passes
        reps = int(np.ceil(budget_s / 2 / t))
        t0 = time.perf_counter()
        for _ in range(reps):
            run(n)
        t = (time.perf_counter() - t0) / reps
    return {"value": by * n / t / 1e9, "unit": "GB/s", "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": f"{n} of {w.n_seqs} sequences of {w.name} (one query row, all {w.num_q_heads} heads), "
                      f"{t:.1f} s per pass, {reps} pass(es); fp64 numpy, BLAS threads={threads}, "
                      f"host cpus={os.cpu_count()}"}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--only", choices=["all", "prefill", "chunk", "mistral", "decode", "merge", "router"],
                    default="all",
                    help="profiling runs: only the segmented headline prefill, the 128K chunk, the Mistral-7B-shaped "
                         "prefill, segmented decode, the merge or the router")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-kernel", type=int, default=0, choices=[0, 1, 2, 3, 4, 5],
                    help="prefill kernel variant (SEGKV_TUNE_PREFILL_KERNEL); 0 = the library's default")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates rocprofv3 byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_probe:
        n = 1 << 30
        src = torch.zeros(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        sync()
        print(json.dumps({"copy_probe_bytes_read_per_launch": n, "copy_probe_bytes_written_per_launch": n,
                          "launches": 3}))
        return

    from long_context_serving_amd import metrics as M
    from long_context_serving_amd import runner as R
    from long_context_serving_amd import workloads as wl
    from long_context_serving_amd import segkv as S
    S.load_library()
    K, Wm = args.steps, args.warmup
    global PREFILL_KERNEL
    PREFILL_KERNEL = args.prefill_kernel
    full = args.only == "all"
    out = {"metric": METRIC, "n_gpus": 1, "steps": K, "warmup": Wm, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) bf16 Q/K/V; no weights or datasets)"}

    def line(rep, config):
        out.update({"value": rep["value"], "unit": rep["unit"], "ms_per_step": rep["ms_per_step"],
                    "config": config, "roofline": rep["roofline"]})

    headline = wl.LLAMA70B_VARLEN_PREFILL
    if args.only in ("all", "prefill"):
        log(f"inputs {headline.name} lengths {list(headline.kv_lens)}")
        x3 = wl.make_inputs(headline)
        dev3 = R.to_device(headline, x3)
        run3, rep3 = prefill_report(headline, dev3, K, Wm, with_global=full, with_protocol=full)
        run3.close()
        line(rep3, {"workload": headline.name, "global_batch": headline.n_seqs,
                    "seq_lens": list(headline.kv_lens), "num_q_heads": headline.num_q_heads,
                    "num_kv_heads": headline.num_kv_heads, "head_dim": headline.head_dim,
                    "page_size": headline.page_size, "head_windows": "1 global + 7 local W=2048",
                    "visible_flops": rep3["visible_flops"], "parallelism": "none (1 GPU)"})
        out["step_breakdown"] = rep3["step_breakdown"]
        for k in ("all_global", "protocol"):
            if k in rep3:
                out[k] = rep3[k]
        if full:
            log("prefill relocated (headline)")
            run_r, rel = prefill_arm(headline, dev3, K, Wm, deltas=local_head_deltas(headline, RELOCATION_OFFSET))
            run_r.close()
            log(f"  {rel}")
            kr = rel["prefill_kernel_ms"] + rel["combine_kernel_ms"]
            kp = rep3["step_breakdown"]["prefill_kernel_ms"] + rep3["step_breakdown"]["combine_kernel_ms"]
            out["relocation"] = {"offset": RELOCATION_OFFSET, "prefill": {
                "workload": headline.name, "kernel_tflops": rep3["visible_flops"] / (kr * 1e-3) / 1e12,
                "step_tflops": rep3["visible_flops"] / (rel["ms_per_step"] * 1e-3) / 1e12,
                "prefill_kernel_ms": rel["prefill_kernel_ms"], "combine_kernel_ms": rel["combine_kernel_ms"],
                "kernel_time_over_plain": kr / kp}}
        if not args.no_cpu_baseline:
            log("cpu baseline (oracle, headline)")
            out["cpu_baseline"] = cpu_baseline(headline, x3)
        del dev3, x3

    secondary = {}
    for w, key in ((wl.CHUNKED_PREFILL_128K, "chunk"), (wl.MISTRAL7B_PREFILL, "mistral")):
        if not (full or args.only == key):
            continue
        log(f"inputs {w.name}")
        x = wl.make_inputs(w)
        dev = R.to_device(w, x)
        del x
        run, rep = prefill_report(w, dev, K, Wm, with_global=full, with_protocol=full)
        if full and w is wl.MISTRAL7B_PREFILL:
            run.close()
            log("router (token scores + top-k)")
            out["router"] = router_arm(w, dev, K, Wm, M.prefill_flops(w) // 2)
            log(f"  {out['router']}")
        else:
            run.close()
        secondary[w.name] = rep
        if args.only == key:
            line(rep, {"workload": w.name, "global_batch": w.n_seqs, "seq_lens": list(w.kv_lens),
                       "q_lens": list(w.q_lens)})
        del dev
    if secondary:
        out["workloads"] = secondary

    if args.only == "router":
        w = wl.MISTRAL7B_PREFILL
        dev = R.to_device(w, wl.make_inputs(w))
        m = router_arm(w, dev, K, Wm, M.prefill_flops(w) // 2)
        out["router"] = m
        out.update({"value": m["roofline"]["achieved"], "unit": "TFLOP/s", "ms_per_step": m["ms_per_call"],
                    "config": {"workload": m["workload"]}, "roofline": m["roofline"]})
        del dev

    if args.only in ("all", "decode"):
        dw = wl.DECODE_32K
        log(f"inputs {dw.name}")
        x4 = wl.make_inputs(dw)
        dev4 = R.to_device(dw, x4)
        by = M.decode_bytes(dw)
        by_g = M.decode_bytes(dw, windows=(0,) * dw.num_kv_heads)
        log("decode segmented")
        d = decode_arm(dw, dev4, K, Wm)
        log(f"  {d}")
        dg = dr = None
        if full:
            log("decode all-global")
            dg = decode_arm(dw, dev4, K, Wm, windows=(0,) * dw.num_kv_heads)
            log(f"  {dg}")
            log("decode relocated")
            dr = decode_arm(dw, dev4, K, Wm, deltas=local_head_deltas(dw, RELOCATION_OFFSET))
            log(f"  {dr}")
        kern = d["split_kernel_ms"] + d["combine_kernel_ms"]
        dec = {
            "metric": "visible-KV GB/s (decode)", "unit": "GB/s", "workload": dw.name,
            "value": by["total"] / (kern * 1e-3) / 1e9,
            "value_step": by["total"] / (d["ms_per_step"] * 1e-3) / 1e9,
            "visible_bytes": by,
            "roofline": {"bound": "hbm", "achieved": by["total"] / (kern * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": by["total"] / (kern * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "traffic": measured_traffic("decode_" + dw.name),
                         "kernel": "decode_kernel<128,64> + combine_kernel<128>",
                         "avg_launch_ms": d["split_kernel_ms"], "combine_ms": d["combine_kernel_ms"]},
            "frac_split_only": by["total"] / (d["split_kernel_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "frac_split_plus_combine": by["total"] / (kern * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "detail": d,
        }
        if dg is not None:
            kern_g = dg["split_kernel_ms"] + dg["combine_kernel_ms"]
            dec["all_global"] = {"value": by_g["total"] / (kern_g * 1e-3) / 1e9, "visible_bytes": by_g,
                                 "detail": dg, "segmented_speedup_kernel": kern_g / kern}
        if dr is not None:
            kern_r = dr["split_kernel_ms"] + dr["combine_kernel_ms"]
            out.setdefault("relocation", {"offset": RELOCATION_OFFSET})["decode"] = {
                "value": by["total"] / (kern_r * 1e-3) / 1e9, "unit": "GB/s", "detail": dr,
                "kernel_time_over_plain": kern_r / kern}
        if not args.no_cpu_baseline:
            log("cpu baseline (oracle, decode)")
            dec["cpu_baseline"] = cpu_baseline_decode(dw, x4)
        out["decode"] = dec
        del dev4, x4
        if full:
            log("decode over forks")
            out["fork"] = fork_arm(dw, K, Wm, d["pages_in_use"])
            log(f"  {out['fork']}")
        if args.only == "decode":
            out.update({"value": dec["value"], "unit": "GB/s", "ms_per_step": d["ms_per_step"],
                        "config": {"workload": dw.name}, "roofline": dec["roofline"]})

    if args.only in ("all", "merge"):
        log(f"merge {wl.MERGE_128K.name}")
        m = merge_arm(wl.MERGE_128K, K, Wm)
        out["merge"] = m
        log(f"  {m['value']:.1f} GB/s, kernel {m['kernel_ms']:.4f} ms")
        if args.only == "merge":
            out.update({"value": m["value"], "unit": "GB/s", "ms_per_step": m["ms_per_call"],
                        "config": {"workload": m["workload"]}, "roofline": m["roofline"]})

    out.setdefault("cpu_baseline", None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
