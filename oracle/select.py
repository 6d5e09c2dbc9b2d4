"""Block selection for block-sparse prefill, step by step (test infrastructure).

Follows the patty.io review of "RBS-Attention: Radius-Bounded Sparse Prefill for
Long-Context LLMs" in the order its sections give the steps:

1. Keys are grouped into blocks and each block is represented by its centroid (the
   mean key); a block's mean score is the query's dot product with that centroid
   (section "the wish to compute less attention is old").  Queries are grouped into
   blocks of the same size and represented by their mean.
2. The rescue signal is the block's maximum key radius: the distance from the
   centroid to the farthest key in the block (section "why bring in the radius").
3. Each signal is thresholded against its own distribution per prompt and per head,
   not against a fixed constant (same section), independently of the other
   (section "what is left when two sieves overlap").
4. The two selections are OR'd into one block mask (same section), which a regular
   block-sparse attention then executes (section "how regular sparsity persuades
   the GPU").

Readings where the page leaves a step open (each is also listed with the design):

* Query block qb = rows [qb*bs, (qb+1)*bs) of the Tq-row block; key block kb =
  absolute keys [kb*bs, (kb+1)*bs) clipped to Tk_b; a short last block averages over
  its actual members.
* Only admissible pairs (qb, kb) -- those holding at least one (row, key) pair the
  position rule allows -- are scored or kept.
* Score s1 = qmean . centroid, unscaled.  Radius kept squared (rad2).  Both are
  monotone transforms, so the selection is the same as with scale or sqrt.
* Threshold = order statistic: with N the population and n = floor(rho*N + 1/2),
  tau = the (n+1)-th largest value, or -inf when n >= N; a block is kept iff its
  value is strictly greater than tau.  Population: the admissible pairs of (b, h)
  for the mean branch; the key blocks of (b, kv head) for the radius branch.
* The radius branch keeps the whole key-block column: every admissible query block
  of every query head that reads that KV head.
* mask = admissible and (s1 > tau1[b, h] or rad2[b, h // g, kb] > tau2[b, h // g]).
* When a keep fraction is negative, the caller's threshold is used as given.
"""
from __future__ import annotations

import math

import numpy as np

from .attend import _f64, _i64


def n_blocks(n, bs):
    return (n + bs - 1) // bs


def block_means(x, n, bs):
    """Mean of rows [i*bs, min((i+1)*bs, n)) of x[:n] for each block i, float64."""
    nb = n_blocks(n, bs)
    out = np.empty((nb, x.shape[-1]))
    for i in range(nb):
        lo, hi = i * bs, min((i + 1) * bs, n)
        out[i] = x[lo:hi].sum(axis=0) / (hi - lo)
    return out


def block_radius2(x, n, bs, centroids):
    """Largest squared distance from the block centroid to a key of the block."""
    nb = n_blocks(n, bs)
    out = np.empty(nb)
    for i in range(nb):
        lo, hi = i * bs, min((i + 1) * bs, n)
        diff = x[lo:hi] - centroids[i][None, :]
        out[i] = (diff * diff).sum(axis=1).max()
    return out


def admissible(tq, tkb, off, window, bs):
    """[nQB, nKB] bool: does the block pair hold at least one allowed (row, key) pair?

    Positions of query block qb run over p0..p1 and its keys j0..j1 (both contiguous);
    the keys any of these rows may see form the interval (p0 - W, p1] (no lower bound
    without a window), so the pair is admissible iff that interval meets [j0, j1].
    """
    nqb, nkb = n_blocks(tq, bs), n_blocks(tkb, bs)
    qb = np.arange(nqb)
    p0 = off + qb * bs
    p1 = off + np.minimum((qb + 1) * bs, tq) - 1
    kb = np.arange(nkb)
    j0 = kb * bs
    j1 = np.minimum((kb + 1) * bs, tkb) - 1
    ok = j0[None, :] <= p1[:, None]
    if window and window > 0:
        ok &= j1[None, :] > (p0 - window)[:, None]
    return ok


def order_statistic_threshold(values, keep_frac):
    """tau such that keeping values > tau keeps the round(keep_frac*N) largest (ties dropped)."""
    N = len(values)
    n = int(math.floor(keep_frac * N + 0.5))
    if n >= N:
        return -np.inf
    return float(np.sort(values)[::-1][n])


def select_blocks(q, k, block_size, cache_off=None, window=0, keep_mean=0.05, keep_radius=0.05,
                  tau_mean=None, tau_radius=None):
    """Block mask from the mean-centroid branch OR the max-radius branch.

    q: [B, Hq, Tq, d]; k: [B, Hkv, Tcap, d].  Returns a dict with
      mask  uint8 [B, Hq, nQB, nKBcap]  (nKBcap = ceil(Tcap/bs); blocks beyond Tk_b are 0)
      adm   bool  [B, nQB, nKBcap]
      qmean float64 [B, Hq, nQB, d]; centroid [B, Hkv, nKBcap, d]; rad2 [B, Hkv, nKBcap]
      score float64 [B, Hq, nQB, nKBcap] (-inf where not admissible)
      tau_mean [B, Hq], tau_radius [B, Hkv]
    A negative keep fraction means the matching tau_* argument ([B,Hq] / [B,Hkv]) is used.
    """
    q, k = _f64(q), _f64(k)
    B, Hq, Tq, d = q.shape
    Hkv, Tcap = k.shape[1], k.shape[2]
    g = Hq // Hkv
    bs = int(block_size)
    off = np.full(B, Tcap - Tq, dtype=np.int64) if cache_off is None else _i64(cache_off)
    nqb, nkbc = n_blocks(Tq, bs), n_blocks(Tcap, bs)

    mask = np.zeros((B, Hq, nqb, nkbc), dtype=np.uint8)
    adm_all = np.zeros((B, nqb, nkbc), dtype=bool)
    qmean = np.zeros((B, Hq, nqb, d))
    cent = np.zeros((B, Hkv, nkbc, d))
    rad2 = np.full((B, Hkv, nkbc), -np.inf)
    score = np.full((B, Hq, nqb, nkbc), -np.inf)
    tau1 = np.zeros((B, Hq))
    tau2 = np.zeros((B, Hkv))
    for b in range(B):
        tkb = int(off[b]) + Tq
        nkb = n_blocks(tkb, bs)
        adm = admissible(Tq, tkb, int(off[b]), window, bs)
        adm_all[b, :, :nkb] = adm
        for kvh in range(Hkv):
            c = block_means(k[b, kvh], tkb, bs)
            cent[b, kvh, :nkb] = c
            rad2[b, kvh, :nkb] = block_radius2(k[b, kvh], tkb, bs, c)
            tau2[b, kvh] = (order_statistic_threshold(rad2[b, kvh, :nkb], keep_radius)
                            if keep_radius >= 0 else float(_f64(tau_radius)[b, kvh]))
        for h in range(Hq):
            kvh = h // g
            qm = block_means(q[b, h], Tq, bs)
            qmean[b, h] = qm
            s = qm @ cent[b, kvh, :nkb].T
            s = np.where(adm, s, -np.inf)
            score[b, h, :, :nkb] = s
            tau1[b, h] = (order_statistic_threshold(s[adm], keep_mean)
                          if keep_mean >= 0 else float(_f64(tau_mean)[b, h]))
            keep = adm & ((s > tau1[b, h]) | (rad2[b, kvh, :nkb] > tau2[b, kvh])[None, :])
            mask[b, h, :, :nkb] = keep
    return dict(mask=mask, adm=adm_all, qmean=qmean, centroid=cent, rad2=rad2, score=score,
                tau_mean=tau1, tau_radius=tau2)


def block_list_from_mask(mask):
    """Kept key blocks per (b, h, qb) in ascending order: int32 [..., 1 + nKB] = count, indices."""
    m = np.asarray(mask) != 0
    out = np.zeros(m.shape[:-1] + (m.shape[-1] + 1,), dtype=np.int32)
    for idx in np.ndindex(*m.shape[:-1]):
        kept = np.nonzero(m[idx])[0]
        out[idx][0] = len(kept)
        out[idx][1:1 + len(kept)] = kept
    return out
