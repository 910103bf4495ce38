"""Pure-Python brute-force attention for pinning the oracle on tiny inputs.

Written separately from ``oracle/attention.py`` (no numpy vectorisation, no
masks, no blocking), straight from the visibility reading: key j is visible
to the query at position p iff j <= p and, for a local head of window W,
j > p - W.  Query t of a sequence with kv_len keys and q_len queries sits at
kv_len - q_len + t; query head h uses KV head h // (Hq / Hkv).
"""

import math

import numpy as np


def brute_attention(q, k, v, kv_len, windows, scale):
    """Pure-Python reference written from the visibility reading:
    key j is visible to a query at p iff j <= p and (W == 0 or j > p - W)."""
    q_len, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    o = np.zeros((q_len, hq, d))
    lse = np.zeros((q_len, hq))
    for t in range(q_len):
        p = kv_len - q_len + t
        for h in range(hq):
            g = h // grp
            w = windows[g]
            js = [j for j in range(kv_len) if j <= p and (w == 0 or j > p - w)]
            s = [scale * sum(q[t, h, c] * k[j, g, c] for c in range(d)) for j in js]
            mx = max(s)
            ex = [math.exp(x - mx) for x in s]
            tot = sum(ex)
            lse[t, h] = mx + math.log(tot)
            for c in range(d):
                o[t, h, c] = sum(e * v[j, g, c] for e, j in zip(ex, js)) / tot
    return o, lse
