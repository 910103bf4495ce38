#!/usr/bin/env python3
"""Benchmark of segmented paged attention on one MI355X.

One step = one pass of the attention hot path over one batch of the
workload: release the batch's sequences, append their cache fill (no
queries) and their query tokens (page allocation, table upload, KV
scatter), then run varlen prefill.  Inputs are resident in HBM before the
timed region.

Headline: the Mistral-7B-shaped layer prefill (1 sequence, L = 8192, 32
query / 8 KV heads, D = 128, 1 global + 7 local KV heads with W = 1024,
page 64, random page order).  value = visible-token TFLOP/s = 4 * D *
(visible (query head, query, key) pairs) per step / step time.

In the same JSON line:
  roofline      the prefill kernel's rate from HIP events recorded around
                each launch on the library's stream, against the 2.5 PFLOP/s
                dense bf16 MFMA peak (traffic: rocprofv3 counter bytes when
                they were taken on the current kernel source, else null);
  all_global    the same steps with every head forced global;
  relocation    query-side RoPE relocation: the same prefill and decode with
                every local head's queries relocated by a document offset
                (the global head at offset 0), and the cost over the plain
                kernels;
  protocol      3 unmeasured + 10 measured (segmented, all-global) pairs,
                p50 / p95 of the prefill kernel time;
  decode        visible-KV GB/s of split-KV decode + combine at 32K x 31
                sequences against 8 TB/s, and its all-global arm;
  router        attention-mass token scores of the headline prefill (a second
                MFMA pass over the visible pairs, QK only: 2 D FLOPs per pair)
                and the top-k (k = L/4) that routes tokens to the dense FFN;
  merge         the head-decomposition merge of a reused 128K-token document
                (offline Local-head partials, online Global heads and
                protected rows, LSE merge on the window's boundary rows):
                algorithmic GB/s against 8 TB/s;
  fork          copy-on-write forks: the 32K x 31 decode with the 31 sequences
                forked from one 32767-token parent (each appends its own query
                token): pages in use against 31 unshared copies, forks that fit
                in the unshared pool, and the decode kernel over the forks;
  workloads     the varlen Llama-3.3-70B-shaped and the 128K chunked prefill;
  cpu_baseline  the fp64 oracle on a bounded sample of the headline workload.

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
KERNEL_SRC = os.path.join(ROOT, "long_context_serving_amd", "csrc", "kernels.hip")
RELOCATION_OFFSET = 8192    # document offset of the relocation arm


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(key)
    if not e or e.get("kernel_source_sha256_16") != kernel_source_hash():
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

def prefill_arm(w, dev, steps, warmup, windows=None, split_tiles=None, deltas=None):
    import torch
    from long_context_serving_amd import runner as R
    from long_context_serving_amd import segkv as S
    run = R.WorkloadRun(w, dev, windows=windows, deltas=deltas)
    if split_tiles:
        run.ctx.set_tuning(S.TUNE_PREFILL_SPLIT_TILES, split_tiles)
    o = torch.empty_like(dev.q)
    lse = torch.empty(dev.q.shape[:2], dtype=torch.float32, device=dev.q.device)

    def step():
        run.reset()
        run.load()
        run.prefill(o, lse)

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
    c_ms, _ = kernel_avg(run.ctx, S.KERNEL_COMBINE)
    run.ctx.set_timing(True, [S.KERNEL_SCATTER])
    for _ in range(max(2, steps // 4)):
        step()
    sync()
    s_ms, s_n = kernel_avg(run.ctx, S.KERNEL_SCATTER)
    run.ctx.set_timing(False)
    return run, {"ms_per_step": dt * 1e3, "prefill_kernel_ms": k_ms, "prefill_launches": k_n,
                 "combine_kernel_ms": c_ms, "scatter_kernel_ms_per_launch": s_ms,
                 "scatter_launches_per_step": s_n / max(max(2, steps // 4), 1)}


def paired_protocol(run_a, run_b, warm=3, measured=10):
    """The pages' timing protocol at kernel level: unmeasured warm pairs, then
    measured (segmented, all-global) pairs; returns per-arm kernel times."""
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


# ---------------------------------------------------------------- decode

def decode_arm(w, dev, steps, warmup, windows=None, deltas=None):
    import torch
    from long_context_serving_amd import runner as R
    from long_context_serving_amd import segkv as S
    run = R.WorkloadRun(w, dev, windows=windows, deltas=deltas).load()
    o = torch.empty_like(dev.q)
    lse = torch.empty(dev.q.shape[:2], dtype=torch.float32, device=dev.q.device)
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
    for _ in range(warmup):
        run.ctx.token_scores(0, run.seq_ids, w.q_lens, dev.q, lse, scores)
        run.ctx.topk(w.q_lens, scores, k, idx)
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
                         "frac": tf / PEAK_BF16_TFLOPS, "traffic": None, "kernel": "score_kernel<128,64>",
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


def cpu_baseline(w, x, budget_s=15.0):
    """The fp64 oracle, as it stands, on a seeded sample of query rows of the
    workload (all heads), timed on the host cores."""
    from oracle import attention as A
    from long_context_serving_amd import metrics as M
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    rng = np.random.default_rng(2024)
    q_len = w.q_lens[0]

    def run(n):
        rows = np.sort(rng.choice(q_len, size=min(n, q_len), replace=False))
        t0 = time.perf_counter()
        A.attend_batch(x.q, x.k, x.v, x.cu_q, x.cu_kv, w.windows, w.scale, rows_per_seq=[rows])
        return time.perf_counter() - t0, M.prefill_flops_rows(w, 0, rows), len(rows)

    n = 64
    t, flops, n = run(n)
    while t < budget_s / 3 and n < q_len:   # grow the sample until it is ~budget_s of work
        n = int(min(q_len, n * max(2.0, min(8.0, budget_s / max(t, 1e-3)))))
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
           "sample": f"{n} of {q_len} query rows (seeded), all {w.num_q_heads} query heads, of "
                     f"{w.name}; {t:.1f} s per pass, {reps} pass(es); fp64 numpy, BLAS threads={threads}, host cpus={os.cpu_count()}"}
    # The same oracle on one thread, on a smaller sample (about a third of the budget).
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        return out
    with threadpool_limits(limits=1):
        n1 = 16
        t1, f1, n1 = run(n1)
        while t1 < budget_s / 9 and n1 < q_len:
            n1 = int(min(q_len, n1 * max(2.0, min(8.0, budget_s / 3 / max(t1, 1e-3)))))
            t1, f1, n1 = run(n1)
    out["single_thread"] = {"value": f1 / t1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                            "sample": f"{n1} of {q_len} query rows (seeded), {t1:.1f} s"}
    return out


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU reaches its steady clock after ~100 headline steps (~40 ms of
    # work) and drops back within a second of idling, so every arm warms up
    # with its own W untimed steps.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "merge", "router"], default="all",
                    help="profiling runs: only the segmented headline prefill, or only segmented decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the varlen and 128K prefill workloads")
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
    from long_context_serving_amd import segkv as S
    from long_context_serving_amd import workloads as wl
    S.load_library()
    K, Wm = args.steps, args.warmup
    out = {}

    headline = wl.MISTRAL7B_PREFILL
    flops = M.prefill_flops(headline)
    flops_g = M.prefill_flops(headline, windows=(0,) * headline.num_kv_heads)
    if args.only in ("all", "prefill"):
        log(f"inputs {headline.name}")
        x2 = wl.make_inputs(headline)
        dev2 = R.to_device(headline, x2)
        log("prefill segmented")
        run_seg, seg = prefill_arm(headline, dev2, K, Wm)
        log(f"  {seg}")
        if args.only == "all":
            log("prefill all-global")
            run_glob, glob = prefill_arm(headline, dev2, K, Wm, windows=(0,) * headline.num_kv_heads)
            log(f"  {glob}")
            proto = paired_protocol(run_seg, run_glob)
            run_glob.close()
            log("router (token scores + top-k)")
            out["router"] = router_arm(headline, dev2, K, Wm, flops // 2)
            log(f"  {out['router']}")
            log("prefill relocated")
            run_rel, rel = prefill_arm(headline, dev2, K, Wm, deltas=local_head_deltas(headline, RELOCATION_OFFSET))
            run_rel.close()
            log(f"  {rel}")
        run_seg.close()
        achieved = flops / (seg["prefill_kernel_ms"] * 1e-3) / 1e12
        traffic = measured_traffic("prefill_" + headline.name)
        out.update({
            "metric": METRIC, "value": flops / (seg["ms_per_step"] * 1e-3) / 1e12, "unit": "TFLOP/s",
            "n_gpus": 1, "steps": K, "warmup": Wm, "ms_per_step": seg["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16 Q/K/V; no weights or datasets)",
            "config": {"workload": headline.name, "global_batch": 1, "seq_len": 8192, "num_q_heads": 32,
                       "num_kv_heads": 8, "head_dim": 128, "page_size": 64,
                       "head_windows": "1 global + 7 local W=1024", "visible_flops": flops,
                       "parallelism": "none (1 GPU)"},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                         "kernel": "prefill_kernel<128,64>", "avg_launch_ms": seg["prefill_kernel_ms"]},
            "step_breakdown": seg,
        })
        if args.only == "all":
            out.update({
            "all_global": {"value": flops_g / (glob["ms_per_step"] * 1e-3) / 1e12, "unit": "TFLOP/s",
                           "visible_flops": flops_g, "ms_per_step": glob["ms_per_step"],
                           "prefill_kernel_ms": glob["prefill_kernel_ms"],
                           "kernel_tflops": flops_g / (glob["prefill_kernel_ms"] * 1e-3) / 1e12,
                           "segmented_speedup_step": glob["ms_per_step"] / seg["ms_per_step"],
                           "segmented_speedup_kernel": glob["prefill_kernel_ms"] / seg["prefill_kernel_ms"]},
            "protocol": proto,
            "relocation": {"offset": RELOCATION_OFFSET, "prefill": {
                "kernel_tflops": flops / (rel["prefill_kernel_ms"] * 1e-3) / 1e12,
                "step_tflops": flops / (rel["ms_per_step"] * 1e-3) / 1e12,
                "prefill_kernel_ms": rel["prefill_kernel_ms"],
                "kernel_time_over_plain": rel["prefill_kernel_ms"] / seg["prefill_kernel_ms"]}},
        })
        del dev2

    if args.only == "router":
        log(f"inputs {headline.name}")
        dev2 = R.to_device(headline, wl.make_inputs(headline))
        out["router"] = router_arm(headline, dev2, K, Wm, flops // 2)
        del dev2

    if args.only in ("all", "decode"):
        dw = wl.DECODE_32K
        log(f"inputs {dw.name}")
        x4 = wl.make_inputs(dw)
        dev4 = R.to_device(dw, x4)
        del x4
        by = M.decode_bytes(dw)
        by_g = M.decode_bytes(dw, windows=(0,) * dw.num_kv_heads)
        log("decode segmented")
        d = decode_arm(dw, dev4, K, Wm)
        log(f"  {d}")
        dg = dr = None
        if args.only == "all":
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
            "roofline": {"bound": "hbm", "achieved": by["total"] / (d["split_kernel_ms"] * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": by["total"] / (d["split_kernel_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "traffic": measured_traffic("decode_" + dw.name),
                         "kernel": "decode_kernel<128,64>", "avg_launch_ms": d["split_kernel_ms"]},
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
        out["decode"] = dec
        del dev4
        if args.only == "all":
            log("decode over forks")
            out["fork"] = fork_arm(dw, K, Wm, d["pages_in_use"])
            log(f"  {out['fork']}")

    if args.only in ("all", "merge"):
        log(f"merge {wl.MERGE_128K.name}")
        out["merge"] = merge_arm(wl.MERGE_128K, K, Wm)
        log(f"  {out['merge']['value']:.1f} GB/s, kernel {out['merge']['kernel_ms']:.4f} ms")

    if args.only == "all" and not args.no_secondary:
        sec = {}
        for w, split in ((wl.LLAMA70B_VARLEN_PREFILL, None), (wl.CHUNKED_PREFILL_128K, None)):
            log(f"inputs {w.name}")
            x = wl.make_inputs(w)
            dev = R.to_device(w, x)
            del x
            f = M.prefill_flops(w)
            steps = max(2, K // 8)
            run, r = prefill_arm(w, dev, steps, max(1, Wm // 8), split_tiles=split)
            run.close()
            sec[w.name] = {"visible_flops": f, "steps": steps, "step_tflops": f / (r["ms_per_step"] * 1e-3) / 1e12,
                           "kernel_tflops": f / ((r["prefill_kernel_ms"] + r["combine_kernel_ms"]) * 1e-3) / 1e12,
                           "frac_of_peak": f / ((r["prefill_kernel_ms"] + r["combine_kernel_ms"]) * 1e-3) / 1e12
                           / PEAK_BF16_TFLOPS, "detail": r}
            log(f"  {sec[w.name]}")
            del dev
        out["workloads"] = sec

    if args.only in ("all", "prefill") and not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(headline, wl.make_inputs(headline))
    elif "value" in out:
        out["cpu_baseline"] = None

    if "value" not in out and args.only == "router":  # profiling runs still print one line
        m = out["router"]
        out = {"metric": METRIC, "value": m["roofline"]["achieved"], "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
               "warmup": Wm, "ms_per_step": m["ms_per_call"], "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": {"workload": m["workload"]},
               "roofline": m["roofline"], "cpu_baseline": None, "router": m}
    if "value" not in out and args.only == "merge":  # profiling runs still print one line
        m = out["merge"]
        out = {"metric": METRIC, "value": m["value"], "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": Wm,
               "ms_per_step": m["ms_per_call"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
               "dtype": "bf16", "data": "synthetic", "config": {"workload": m["workload"]},
               "roofline": m["roofline"], "cpu_baseline": None, "merge": m}
    if "value" not in out:  # decode-only runs still print one line
        dec = out.get("decode", {})
        out = {"metric": METRIC, "value": dec.get("value"), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": Wm,
               "ms_per_step": dec.get("detail", {}).get("ms_per_step"), "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
               "config": {"workload": wl.DECODE_32K.name}, "roofline": dec.get("roofline"), "cpu_baseline": None,
               "decode": dec}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
