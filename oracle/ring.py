"""A W-slot ring-buffer KV cache (test infrastructure).

Follows sotaaz.com/post/attention-in-code, section 2 ("Sliding window: ring
buffer"): a layer that only looks at the last W tokens keeps W slots per KV
head; token number n is written into slot n mod W, overwriting the oldest one,
and attention runs over the filled slots with no mask at all, because a softmax
over a set of keys does not depend on their order.

It is an independent route to the window rule: attention over the ring's
contents must equal masked attention with window W at every step.
"""
from __future__ import annotations

import math

import numpy as np


class RingCache:
    def __init__(self, n_kv, head_dim, window):
        self.k = np.zeros((n_kv, window, head_dim))
        self.v = np.zeros((n_kv, window, head_dim))
        self.w = window
        self.n = 0  # tokens written so far

    def add(self, k_new, v_new):
        """k_new, v_new: [n_kv, d] for one token.  Returns the filled slots (unordered)."""
        slot = self.n % self.w
        self.k[:, slot] = k_new
        self.v[:, slot] = v_new
        self.n += 1
        filled = min(self.n, self.w)
        return self.k[:, :filled], self.v[:, :filled]


def attend_unmasked(q_row, K, V, n_heads, sink=None, scale=None):
    """One query token's heads over a key set with no mask.

    q_row: [Hq, d]; K, V: [Hkv, n, d]; head h reads KV head h // (Hq/Hkv).
    """
    Hkv = K.shape[0]
    g = n_heads // Hkv
    d = q_row.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.zeros((n_heads, V.shape[-1]))
    for h in range(n_heads):
        s = scale * (K[h // g] @ q_row[h])
        top = s.max() if sink is None else max(s.max(), sink[h])
        w = np.exp(s - top)
        z = w.sum() + (0.0 if sink is None else math.exp(sink[h] - top))
        out[h] = (w @ V[h // g]) / z
    return out
