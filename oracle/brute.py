"""Scalar brute force for tiny shapes (test infrastructure).

A second, independent implementation of the attention definition and of block
selection, written as explicit Python loops over every index with ``math.exp``;
it shares nothing with the vectorised oracle beyond the definitions themselves
(sotaaz.com/post/attention-in-code, listing ``attend``/``causal`` and sections 1
and 3; patty.io RBS-Attention review, sections on the centroid score, the
radius and the two thresholds).  Only for shapes of a few dozen tokens.
"""
from __future__ import annotations

import math


def _tolist(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch

        return x.detach().cpu().to(torch.float64).tolist()
    return x.tolist() if hasattr(x, "tolist") else x


def _visible(pos, j, window):
    if j > pos:
        return False
    if window > 0 and j <= pos - window:
        return False
    return True


def attend_brute(q, k, v, cache_off=None, window=0, sink=None, scale=None, block_mask=None,
                 block_size=0):
    q, k, v, sink = _tolist(q), _tolist(k), _tolist(v), _tolist(sink)
    bm = _tolist(block_mask)
    B, Hq, Tq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Tcap = len(k[0]), len(k[0][0])
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    offs = [Tcap - Tq] * B if cache_off is None else [int(x) for x in _tolist(cache_off)]
    out = [[[[0.0] * d for _ in range(Tq)] for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        tkb = offs[b] + Tq
        for h in range(Hq):
            kv = h // g
            for r in range(Tq):
                pos = offs[b] + r
                logits = []
                for j in range(tkb):
                    if not _visible(pos, j, window):
                        continue
                    if bm is not None and not bm[b][h][r // block_size][j // block_size]:
                        continue
                    dot = 0.0
                    for t in range(d):
                        dot += q[b][h][r][t] * k[b][kv][j][t]
                    logits.append((j, scale * dot))
                cands = [s for _, s in logits] + ([sink[h]] if sink is not None else [])
                if not cands or max(cands) == -math.inf:
                    continue
                top = max(cands)
                z = sum(math.exp(s - top) for s in cands)
                for j, s in logits:
                    w = math.exp(s - top) / z
                    for t in range(d):
                        out[b][h][r][t] += w * v[b][kv][j][t]
    return out


def select_brute(q, k, block_size, cache_off=None, window=0, keep_mean=0.05, keep_radius=0.05):
    """Returns (mask[b][h][qb][kb] as 0/1 over kb < ceil(Tcap/bs), tau_mean, tau_radius)."""
    q, k = _tolist(q), _tolist(k)
    B, Hq, Tq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Tcap = len(k[0]), len(k[0][0])
    g = Hq // Hkv
    bs = block_size
    offs = [Tcap - Tq] * B if cache_off is None else [int(x) for x in _tolist(cache_off)]
    nqb = -(-Tq // bs)
    nkbc = -(-Tcap // bs)
    mask = [[[[0] * nkbc for _ in range(nqb)] for _ in range(Hq)] for _ in range(B)]
    taus1 = [[0.0] * Hq for _ in range(B)]
    taus2 = [[0.0] * Hkv for _ in range(B)]

    def mean_rows(rows):
        return [sum(row[t] for row in rows) / len(rows) for t in range(d)]

    def kth_largest_threshold(vals, frac):
        n = int(math.floor(frac * len(vals) + 0.5))
        if n >= len(vals):
            return -math.inf
        return sorted(vals, reverse=True)[n]

    for b in range(B):
        tkb = offs[b] + Tq
        nkb = -(-tkb // bs)
        adm = [[False] * nkb for _ in range(nqb)]
        for qb in range(nqb):
            for kb in range(nkb):
                for r in range(qb * bs, min((qb + 1) * bs, Tq)):
                    for j in range(kb * bs, min((kb + 1) * bs, tkb)):
                        if _visible(offs[b] + r, j, window):
                            adm[qb][kb] = True
        cents, rads = [], []
        for kv in range(Hkv):
            c_kv, r_kv = [], []
            for kb in range(nkb):
                rows = k[b][kv][kb * bs:min((kb + 1) * bs, tkb)]
                c = mean_rows(rows)
                c_kv.append(c)
                r_kv.append(max(sum((row[t] - c[t]) ** 2 for t in range(d)) for row in rows))
            cents.append(c_kv)
            rads.append(r_kv)
            taus2[b][kv] = kth_largest_threshold(r_kv, keep_radius)
        for h in range(Hq):
            kv = h // g
            qm = [mean_rows(q[b][h][qb * bs:min((qb + 1) * bs, Tq)]) for qb in range(nqb)]
            scores = {}
            for qb in range(nqb):
                for kb in range(nkb):
                    if adm[qb][kb]:
                        scores[(qb, kb)] = sum(qm[qb][t] * cents[kv][kb][t] for t in range(d))
            tau = kth_largest_threshold(list(scores.values()), keep_mean)
            taus1[b][h] = tau
            for (qb, kb), s in scores.items():
                if s > tau or rads[kv][kb] > taus2[b][kv]:
                    mask[b][h][qb][kb] = 1
    return mask, taus1, taus2
