"""Token top-k sparse attention with a lightning-style indexer (test infrastructure).

Follows sotaaz.com/post/attention-in-code, section 5 (sparse attention: keep everything,
read a little).  A small scorer (the indexer) rates every earlier token for the current
query, and attention runs only over the k best-rated ones; the cache itself is not
shrunk.

* Indexer: a few small query heads qi[j] (width di) per query token, one small key ki[s]
  per cached token, and a weight w[j] per head and query token:
      score(t, s) = sum_j w[j, t] * relu(qi[j, t] . ki[s]).
* Kept set of query token t (at position off_b + t): among the tokens it may see under the
  offset-causal rule (s <= off_b + t), the k with the largest score; all of them if fewer
  than k are visible.  Equal scores are ordered by lower token index first (the page's
  top-k leaves the order of equal scores open; this fixes one).
* Output: the plain attention definition (``oracle.attend``: grouped-query sharing, sink,
  scale) restricted to the kept set, which is shared by every head of the query token.

With k at least the number of visible tokens the kept set is every visible token and the
result is dense attention exactly (the pages report a difference of 0).

Shapes: q [B, Hq, Tq, d], k, v [B, Hkv, Tcap, d]; qi [B, Hi, Tq, di], ki [B, Tcap, di],
wi [B, Hi, Tq].
"""
from __future__ import annotations

import numpy as np

from .attend import _f64, _i64, attend


def indexer_scores(qi, ki, wi):
    """score[b, t, s] = sum_j wi[b, j, t] * relu(qi[b, j, t] . ki[b, s]), float64 [B, Tq, Tcap]."""
    QI, KI, WI = _f64(qi), _f64(ki), _f64(wi)
    dots = np.einsum("bjtd,bsd->bjts", QI, KI)
    return np.einsum("bjt,bjts->bts", WI, np.maximum(dots, 0.0))


def topk_keep(scores, k, cache_off=None):
    """Boolean [B, Tq, Tcap]: the kept set of every query token (see the module text)."""
    S = np.asarray(scores, dtype=np.float64)
    B, Tq, Tcap = S.shape
    off = np.full(B, Tcap - Tq, dtype=np.int64) if cache_off is None else _i64(cache_off)
    keep = np.zeros((B, Tq, Tcap), dtype=bool)
    for b in range(B):
        for t in range(Tq):
            n_vis = int(off[b]) + t + 1
            vis = np.arange(n_vis)
            # sort by score descending, then token index ascending
            order = np.lexsort((vis, -S[b, t, :n_vis]))
            keep[b, t, order[:min(k, n_vis)]] = True
    return keep


def sparse_attend(q, k, v, qi, ki, wi, topk, cache_off=None, sink=None, scale=None, return_keep=False):
    scores = indexer_scores(qi, ki, wi)
    keep = topk_keep(scores, topk, cache_off)
    B, Hq = q.shape[0], q.shape[1]
    mask = np.broadcast_to(keep[:, None], (B, Hq) + keep.shape[1:])  # the same set for every head
    o = attend(q, k, v, cache_off=cache_off, sink=sink, scale=scale, block_mask=mask, block_size=1)
    return (o, keep, scores) if return_keep else o
