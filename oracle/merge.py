"""fp64 oracle of the head-decomposition merge.

TEST INFRASTRUCTURE (see the package docstring of ``oracle``).

RedKnot splits attention heads into Local contributions prepared offline
and Global ones computed online.  It merges the two paths back without
changing the model's interface ("RedKnot: Head-Aware KV Reuse and
SegPagedAttention" page, "The Three Core Mechanisms in Detail", first
mechanism).  RedKnot-MLA also recomputes a protected set of token rows
online: query, new and dirty rows, 128-token boundaries, the indexer's top
rows and a 32K tail.  It states that the factorisation is exact under full
recomputation ("RedKnot-MLA: Multi-Head Offline-Online Reuse for
DeepSeek-V4 Long-Context Serving" review, "Key claims under review" and
"Strengths").

At the level of attention outputs, each (row, query head) therefore takes
one of three results:

* ``TAKE_A``: the offline partial (o_a, lse_a), as stored;
* ``TAKE_B``: the online partial (o_b, lse_b), as computed;
* ``MERGE``: both partials, when they attend to disjoint key sets (e.g. the
  document's own keys offline, the keys before the document online).  The
  softmax over the union of the two key sets is then the log-sum-exp merge:
  lse = ln(e^lse_a + e^lse_b), o = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b.
  A part with lse = -inf has no keys and weighs 0; if both have none, o = 0
  and lse = -inf.

Readings taken where the pages are silent: the mode is given per (row,
head), o is rounded once to bfloat16 by the GPU, and which rows are
protected is the caller's policy.
"""

from __future__ import annotations

import numpy as np

TAKE_A = 0
TAKE_B = 1
MERGE = 2


def merge_pair(o_a, lse_a, o_b, lse_b):
    """Log-sum-exp merge of two partial attentions over disjoint key sets.
    o_*: [..., D]; lse_*: [...]."""
    o_a, o_b = np.asarray(o_a, np.float64), np.asarray(o_b, np.float64)
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    empty = np.isneginf(lse)
    safe = np.where(empty, 0.0, lse)
    wa = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - safe))
    wb = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - safe))
    o = wa[..., None] * o_a + wb[..., None] * o_b
    return np.where(empty[..., None], 0.0, o), lse


def head_decomposition_merge(o_a, lse_a, o_b, lse_b, mode):
    """Per-(row, head) select or merge.  o_*: [rows][heads][D], lse_*:
    [rows][heads], mode: [rows][heads] of TAKE_A / TAKE_B / MERGE."""
    mode = np.asarray(mode)
    if not np.all(np.isin(mode, (TAKE_A, TAKE_B, MERGE))):
        raise ValueError("mode values must be TAKE_A, TAKE_B or MERGE")
    mo, ml = merge_pair(o_a, lse_a, o_b, lse_b)
    o_a, o_b = np.asarray(o_a, np.float64), np.asarray(o_b, np.float64)
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    o = np.where((mode == TAKE_A)[..., None], o_a, np.where((mode == TAKE_B)[..., None], o_b, mo))
    lse = np.where(mode == TAKE_A, lse_a, np.where(mode == TAKE_B, lse_b, ml))
    return o, lse
