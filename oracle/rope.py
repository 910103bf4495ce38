"""fp64 oracle of query-side RoPE relocation.

TEST INFRASTRUCTURE (see the package docstring of ``oracle``).

RedKnot-MLA prefills each reusable document once at canonical position zero.
When the document sits at offset delta in a live request, it rotates the
queries by the negative position offset and does not re-encode the stored
keys ("RedKnot-MLA: Multi-Head Offline-Online Reuse for DeepSeek-V4
Long-Context Serving" review, "Summary" and "Frequently asked questions";
the paper page's abstract).  A rotary position code makes q.k depend only on
the position difference.  Scoring a query rotated to p - delta against keys
rotated to j - delta therefore gives the same scores as p against j.

Readings taken where the pages are silent:

* the rotary code acts on the trailing ``rope_dims`` channels of a head
  (all of them by default), and the other channels pass through unchanged.
  This is the split that MLA's rope sub-dimension uses;
* within that block, pair i turns by pos * theta^(-2 i / rope_dims).
  ``style`` 0 is rotate-half, pairing channel i with i + rope_dims/2;
  ``style`` 1 is interleaved, pairing channels 2i and 2i + 1;
* delta is a per-(layer, sequence, KV head) integer; 0 means no
  relocation;
* queries arrive already encoded at their absolute positions, so
  relocation is one more rotation by -delta;
* relocation yields a query in the attention's input type.  The rotation
  is evaluated in fp64 and rounded once to bfloat16 (round to nearest,
  ties to even) before scoring.
"""

from __future__ import annotations

import numpy as np

from . import attention as A


def pair_freqs(rope_dims: int, theta: float) -> np.ndarray:
    """Angular frequency of each of the rope_dims/2 channel pairs."""
    i = np.arange(rope_dims // 2, dtype=np.float64)
    return theta ** (-2.0 * i / rope_dims)


def rope_rotate(x, pos, theta: float, style: int = 0, rope_dims: int = 0) -> np.ndarray:
    """Rotate the last axis (length D) of x by position(s) ``pos``.

    ``pos`` broadcasts against x's leading axes: a scalar, or one position
    per row.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    r = rope_dims or d
    lead = x[..., : d - r]
    blk = x[..., d - r:]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * pair_freqs(r, theta)
    c, s = np.cos(ang), np.sin(ang)
    if style == 0:
        a, b = blk[..., : r // 2], blk[..., r // 2:]
        rot = np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
    elif style == 1:
        a, b = blk[..., 0::2], blk[..., 1::2]
        rot = np.empty_like(blk)
        rot[..., 0::2] = a * c - b * s
        rot[..., 1::2] = a * s + b * c
    else:
        raise ValueError("style must be 0 (rotate-half) or 1 (interleaved)")
    return np.concatenate([np.broadcast_to(lead, rot.shape[:-1] + lead.shape[-1:]), rot], axis=-1)


def round_to_bf16(x) -> np.ndarray:
    """fp64 -> nearest bfloat16 value (ties to even), returned as fp64.
    bfloat16 has an 8-bit significand and fp32's exponent range; subnormal
    results are quantised to multiples of 2^-133."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)  # below 2^-126 the spacing stays 2^-133
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


def relocate_queries(q, delta: int, theta: float, style: int = 0, rope_dims: int = 0) -> np.ndarray:
    """Queries encoded at absolute positions, turned back by delta and
    rounded to bfloat16."""
    if delta == 0:
        return np.asarray(q, dtype=np.float64)
    return round_to_bf16(rope_rotate(q, -float(delta), theta, style, rope_dims))


def attend_sequence_relocated(q, k, v, windows, scale, deltas, theta, style=0, rope_dims=0, rows=None):
    """Attention of one sequence in which the queries of KV head g's group
    are relocated by -deltas[g] before scoring (fp64).  The layouts are those
    of ``attention.attend_sequence``."""
    q = np.array(q, dtype=np.float64, copy=True)
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    for g in range(hkv):
        if deltas[g]:
            hs = slice(g * group, (g + 1) * group)
            q[:, hs, :] = relocate_queries(q[:, hs, :], deltas[g], theta, style, rope_dims)
    return A.attend_sequence(q, k, v, windows, scale, rows=rows)


def attend_batch_relocated(q_bits, k_bits, v_bits, cu_q, cu_kv, windows, scale, deltas_per_seq, theta,
                           style=0, rope_dims=0, rows_per_seq=None):
    """Varlen batch on bf16 bit patterns with per-(sequence, KV head)
    deltas (``deltas_per_seq[b][g]``)."""
    outs = []
    for b in range(len(cu_q) - 1):
        q = A.bf16_bits_to_f64(q_bits[cu_q[b]:cu_q[b + 1]])
        k = A.bf16_bits_to_f64(k_bits[cu_kv[b]:cu_kv[b + 1]])
        v = A.bf16_bits_to_f64(v_bits[cu_kv[b]:cu_kv[b + 1]])
        rows = None if rows_per_seq is None else rows_per_seq[b]
        outs.append(attend_sequence_relocated(q, k, v, windows, scale, deltas_per_seq[b], theta, style,
                                              rope_dims, rows=rows))
    return outs
