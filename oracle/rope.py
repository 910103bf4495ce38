"""fp64 oracle of query-side RoPE relocation.

TEST INFRASTRUCTURE (see the package docstring of ``oracle``).

RedKnot-MLA prefills each reusable document once at canonical position zero
and, when the document sits at offset delta in a live request, rotates the
queries by the negative position offset instead of re-encoding the stored
keys ("RedKnot-MLA: Multi-Head Offline-Online Reuse for DeepSeek-V4
Long-Context Serving" review, "Summary" and "Frequently asked questions").
Because a rotary position code makes q.k depend only on the position
difference, scoring a query rotated to p - delta against keys rotated to
j - delta gives the same scores as p against j.

Readings taken where the pages are silent:

* the rotary code is the rotate-half form: channel d < D/2 pairs with
  channel d + D/2 and the pair turns by pos * theta^(-2 d / D);
* delta is a per-(sequence, KV head) integer; 0 means no relocation;
* queries arrive already encoded at their absolute positions, so
  relocation is one more rotation by -delta.
"""

from __future__ import annotations

import numpy as np

from . import attention as A


def rope_freqs(head_dim: int, theta: float) -> np.ndarray:
    """Angular frequency of each of the D/2 channel pairs."""
    d = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * d / head_dim)


def rope_rotate(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate the last axis (length D) of x by position(s) ``pos``.

    ``pos`` broadcasts against x's leading axes (a scalar, or one position
    per row).  Pair (d, d + D/2) turns by angle pos * theta^(-2d/D).
    """
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_freqs(x.shape[-1], theta)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def relocate_queries(q: np.ndarray, delta: int, theta: float) -> np.ndarray:
    """Queries encoded at absolute positions, turned back by delta."""
    return rope_rotate(q, -float(delta), theta)


def attend_sequence_relocated(q, k, v, windows, scale, deltas, theta, rows=None):
    """Attention of one sequence where the queries of KV head g's group are
    relocated by -deltas[g] before scoring (fp64).  Same layouts as
    ``attention.attend_sequence``."""
    q = np.array(q, dtype=np.float64, copy=True)
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    for g in range(hkv):
        if deltas[g]:
            for h in range(g * group, (g + 1) * group):
                q[:, h, :] = relocate_queries(q[:, h, :], deltas[g], theta)
    return A.attend_sequence(q, k, v, windows, scale, rows=rows)


def attend_batch_relocated(q_bits, k_bits, v_bits, cu_q, cu_kv, windows, scale, deltas_per_seq, theta,
                           rows_per_seq=None):
    """Varlen batch on bf16 bit patterns with per-(sequence, KV head) deltas."""
    outs = []
    for b in range(len(cu_q) - 1):
        q = A.bf16_bits_to_f64(q_bits[cu_q[b]:cu_q[b + 1]])
        k = A.bf16_bits_to_f64(k_bits[cu_kv[b]:cu_kv[b + 1]])
        v = A.bf16_bits_to_f64(v_bits[cu_kv[b]:cu_kv[b + 1]])
        rows = None if rows_per_seq is None else rows_per_seq[b]
        outs.append(attend_sequence_relocated(q, k, v, windows, scale, deltas_per_seq[b], theta, rows=rows))
    return outs
