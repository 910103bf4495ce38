"""fp64 oracle of attention-mass token scores and their top-k.

TEST INFRASTRUCTURE (see the package docstring of ``oracle``).

RedKnot's sparse FFN runs the dense FFN only on the top-k tokens by
attention score; the other tokens take a residual identity path
("attention as a router": "Xiaohongshu Open-Sources RedKnot" page, "What
Happened" item 2 and "Why Sparse FFN Matters for Agent Workloads"; token
importance scores: "RedKnot: Head-Aware KV Reuse and SegPagedAttention"
page, "The Three Core Mechanisms in Detail", second mechanism).

Readings taken where the pages are silent:

* a token's score is the attention mass it receives as a key: the sum, over
  the call's query rows t and all query heads h that can see it, of the
  normalised probability P[t, h, j] = exp(scale q_{t,h}.k_j - lse_{t,h});
  local heads only see keys in their window, as in the attention itself;
* scores are reported for the tokens of the call's query chunk (the rows
  the FFN processes next), that is, keys kv_len - q_len .. kv_len - 1;
* top-k keeps the k highest scores, ties broken towards the lower index,
  and lists the kept token indices in ascending order.
"""

from __future__ import annotations

import numpy as np

from . import attention as A


def token_scores(q, k, windows, scale, all_keys=False):
    """Attention mass received by each key of the query chunk (or by every
    key when all_keys is set): the normalised probabilities P[t, h, j]
    (zero where j is not visible to row t of head h), added up over rows
    one query head at a time so that large inputs fit in memory."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    q_len, hq, _ = q.shape
    kv_len, hkv, _ = k.shape
    group = hq // hkv
    pos = A.query_positions(kv_len, q_len)
    mass = np.zeros(kv_len)
    for h in range(hq):
        g = h // group
        mask = A.visibility_mask(pos, kv_len, windows[g])
        s = np.where(mask, scale * (q[:, h, :] @ k[:, g, :].T), -np.inf)
        s -= s.max(axis=1, keepdims=True)
        np.exp(s, out=s)
        s /= s.sum(axis=1, keepdims=True)
        mass += s.sum(axis=0)
    if all_keys:
        return mass
    return mass[kv_len - q_len:]


def top_k(scores, k: int) -> np.ndarray:
    """Indices of the k highest scores (ties: lower index first), ascending."""
    scores = np.asarray(scores, np.float64)
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))
    return np.array(sorted(order[:k]), dtype=np.int64)
