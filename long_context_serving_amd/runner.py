"""Drive a synthetic workload through libsegkv: upload inputs, append the
cache fill and the query tokens, run prefill or decode.

Only marshalling lives here (tensor placement, index gathers of the input
rows, call order); all attention work is done by the library's kernels.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import segkv as S
from .workloads import Inputs, Workload


def pages_for(w: Workload, windows=None) -> int:
    """A pool large enough to hold every token of every head (all global)."""
    p = w.page_size
    return int(sum(-(-k // p) + 1 for k in w.kv_lens)) * w.num_kv_heads + 16


@dataclass
class DeviceInputs:
    q: "object"        # bf16 [sum q][Hq][D]
    k_fill: "object"   # bf16 [sum fill][Hkv][D]
    v_fill: "object"
    k_q: "object"      # bf16 [sum q][Hkv][D] (the query tokens' own K/V rows)
    v_q: "object"


def to_device(w: Workload, x: Inputs, device="cuda") -> DeviceInputs:
    import torch
    fill = w.fill_lens()
    fill_idx = np.concatenate([np.arange(x.cu_kv[b], x.cu_kv[b] + fill[b]) for b in range(w.n_seqs)]
                              + [np.zeros(0, np.int64)])
    q_idx = np.concatenate([np.arange(x.cu_kv[b] + fill[b], x.cu_kv[b + 1]) for b in range(w.n_seqs)]
                           + [np.zeros(0, np.int64)])
    k = S.bf16_tensor(x.k, device)
    v = S.bf16_tensor(x.v, device)
    fi = torch.from_numpy(fill_idx).to(device)
    qi = torch.from_numpy(q_idx).to(device)
    out = DeviceInputs(S.bf16_tensor(x.q, device), k.index_select(0, fi).contiguous(),
                       v.index_select(0, fi).contiguous(), k.index_select(0, qi).contiguous(),
                       v.index_select(0, qi).contiguous())
    del k, v
    return out


class WorkloadRun:
    """A libsegkv context holding one workload's sequences in layer 0."""

    def __init__(self, w: Workload, dev: DeviceInputs, page_order_seed: Optional[int] = None,
                 windows=None, num_pages: Optional[int] = None, deltas=None, rope_theta: float = 0.0,
                 rope_style: int = 0, rope_dims: int = 0, pools=None):
        """``deltas[b][g]``: query relocation offset of sequence b, KV head g
        (None = no relocation).  ``pools``: (k_pool, v_pool) tensors to use
        instead of allocating them."""
        self.w = w
        self.dev = dev
        self.windows = tuple(w.windows if windows is None else windows)
        self.deltas = None if deltas is None else np.asarray(deltas, dtype=np.int64).reshape(w.n_seqs, w.num_kv_heads)
        self.ctx = S.SegKV(1, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, max(w.n_seqs, 1),
                           num_pages or pages_for(w), self.windows, softmax_scale=w.scale,
                           page_order_seed=w.page_order_seed if page_order_seed is None else page_order_seed,
                           rope_theta=rope_theta, rope_style=rope_style, rope_dims=rope_dims,
                           max_batch_q_tokens=max(1, sum(w.q_lens)),
                           k_pool=None if pools is None else pools[0], v_pool=None if pools is None else pools[1])
        self.seq_ids = list(range(w.n_seqs))

    def append_fill(self):
        fill = self.w.fill_lens()
        if sum(fill) > 0:
            self.ctx.append_pages(0, self.seq_ids, fill, [0] * self.w.n_seqs, self.dev.k_fill, self.dev.v_fill)

    def append_queries(self):
        self.ctx.append_pages(0, self.seq_ids, self.w.q_lens, self.w.q_lens, self.dev.k_q, self.dev.v_q)

    def load(self, after_append=None):
        """Appends the fill and the queries (``after_append(ctx)`` runs after
        each), then sets the relocation offsets."""
        self.append_fill()
        if after_append:
            after_append(self.ctx)
        self.append_queries()
        if after_append:
            after_append(self.ctx)
        if self.deltas is not None:
            for b, s in enumerate(self.seq_ids):
                self.ctx.set_relocation(s, self.deltas[b])
        return self

    def reset(self):
        for s in self.seq_ids:
            self.ctx.release(s)

    def prefill(self, o=None, lse=None):
        return self.ctx.prefill(0, self.seq_ids, self.w.q_lens, self.dev.q, o, lse)

    def decode(self, o=None, lse=None):
        return self.ctx.decode(0, self.seq_ids, self.dev.q, o, lse)

    def close(self):
        self.ctx.close()
