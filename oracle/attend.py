"""Plain float64 definition of offset-causal masked attention (test infrastructure).

Definition followed (sotaaz.com/post/attention-in-code, "LLM에 적용된 다양한 어텐션
방법들 구현하기", section "the one function every design uses": functions ``attend``
and ``causal``; section 1 for grouped-query sharing; section 3 for the sink):

* Query row r of a Tq-row block sits at absolute position pos = off_b + r, where
  off_b = Tk_b - Tq is the number of cache-held tokens before the block.  Key j is
  visible iff j <= pos, and with a window W > 0 also j > pos - W (W keys including
  the query's own).  This is the position rule of the tilnote.io note on the
  Express framework (section "causal attention is a position problem"): masking by
  the block-internal index is only right when the block starts at position 0.
* Query head h reads KV head h // g with g = Hq / Hkv (repeat_interleave grouping).
* s_j = scale * q . k_j with scale = 1/sqrt(d) unless given.
* Masked keys are excluded exactly (probability zero), not given a large negative
  additive value.
* A sink is one extra logit per head, in the same (post-scale) units as s_j, that
  joins the softmax normaliser and carries no value.
* A row with no visible key and no sink outputs zeros.

Every row is computed exactly from this definition; the only structure is that
rows are taken in blocks so the score matrix of one block fits in memory.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: exact widening, then to numpy
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        return x.detach().cpu().to(dtype=__import__("torch").int64).numpy()
    return np.asarray(x, dtype=np.int64)


def key_allowed(pos, j, window):
    """Boolean (broadcast) of the position rule: j <= pos and, if window > 0, j > pos - window."""
    ok = j <= pos
    if window and window > 0:
        ok = ok & (j > pos - window)
    return ok


def allowed_pair_count(tq, tk, window=0, row_block=1024):
    """Number of (row, key) pairs the rule allows for one head (offset tk - tq)."""
    off = tk - tq
    j = np.arange(tk)[None, :]
    total = 0
    for r0 in range(0, tq, row_block):
        pos = off + np.arange(r0, min(tq, r0 + row_block))[:, None]
        total += int(key_allowed(pos, j, window).sum())
    return total


def attend(q, k, v, cache_off=None, window=0, sink=None, scale=None, block_mask=None,
           block_size=0, rows=None, heads=None, batches=None, row_block=1024, return_lse=False):
    """Masked attention, float64.

    q: [B, Hq, Tq, d]; k: [B, Hkv, Tcap, d]; v: [B, Hkv, Tcap, dv] (numpy or torch, any
    float dtype; dv = d except where the value width differs, as for latent attention).
    cache_off: int [B] or None (then off_b = Tcap - Tq).  Tk_b = off_b + Tq <= Tcap;
    rows of k/v at or beyond Tk_b are never read.
    block_mask: [B, Hq, ceil(Tq/bs), ceil(Tcap/bs)] (nonzero = kept) with bs =
    block_size; query block = r // bs (r is the row inside the Tq block), key block =
    j // bs (j is the absolute key index).
    rows / heads / batches: optional subsets to compute (default all).

    Returns o [len(batches), len(heads), len(rows), dv] float64, and with
    ``return_lse`` also lse = log sum_{allowed j} exp(s_j) (no sink; -inf if empty).
    """
    # inputs are widened to float64 slice by slice (exact), so a large cache is never copied whole
    B, Hq, Tq, d = q.shape
    Hkv, Tcap = k.shape[1], k.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("n_heads must be a multiple of n_kv")
    g = Hq // Hkv
    off = np.full(B, Tcap - Tq, dtype=np.int64) if cache_off is None else _i64(cache_off)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sink = _f64(sink)
    bm = None if block_mask is None else np.asarray(
        block_mask.detach().cpu().numpy() if hasattr(block_mask, "detach") else block_mask)
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, dtype=np.int64)
    batches = np.arange(B) if batches is None else np.asarray(batches, dtype=np.int64)

    out = np.zeros((len(batches), len(heads), len(rows), v.shape[-1]))  # value width may differ from d
    lse = np.full((len(batches), len(heads), len(rows)), -np.inf)
    for bi, b in enumerate(batches):
        tkb = int(off[b]) + Tq
        if off[b] < 0 or tkb > Tcap:
            raise ValueError("cache offset out of range")
        jj = np.arange(tkb)
        for hi, h in enumerate(heads):
            kvh = h // g
            K = _f64(k[b, kvh, :tkb])
            V = _f64(v[b, kvh, :tkb])
            Q = _f64(q[b, h])
            for r0 in range(0, len(rows), row_block):
                r = rows[r0:r0 + row_block]
                pos = int(off[b]) + r
                s = scale * (Q[r] @ K.T)
                allow = key_allowed(pos[:, None], jj[None, :], window)
                if bm is not None:
                    allow = allow & (bm[b, h][(r // block_size)[:, None], (jj // block_size)[None, :]] != 0)
                sm = np.where(allow, s, -np.inf)
                m = sm.max(axis=1) if tkb > 0 else np.full(len(r), -np.inf)
                M = np.maximum(m, sink[h]) if sink is not None else m
                Ms = np.where(np.isfinite(M), M, 0.0)
                e = np.where(allow, np.exp(s - Ms[:, None]), 0.0)
                Z = e.sum(axis=1)
                if sink is not None:
                    Z = Z + np.exp(sink[h] - Ms)
                num = e @ V
                safe = np.where(Z > 0, Z, 1.0)
                out[bi, hi, r0:r0 + len(r)] = np.where((Z > 0)[:, None], num / safe[:, None], 0.0)
                if return_lse:
                    ms = np.where(np.isfinite(m), m, 0.0)
                    se = np.where(allow, np.exp(s - ms[:, None]), 0.0).sum(axis=1)
                    with np.errstate(divide="ignore"):
                        lse[bi, hi, r0:r0 + len(r)] = np.where(se > 0, ms + np.log(se), -np.inf)
    return (out, lse) if return_lse else out
