"""Multi-head latent attention, in the plain form and in the absorbed form (test
infrastructure).

Follows sotaaz.com/post/attention-in-code, section 4 (MLA: keep only the latent, move the
weights to the query side).  Per cached token the cache holds a latent c_kv (width r) and
one small key k_rope (width dr) shared by all heads.  Head h's key for a cached token is
the concatenation [c_kv @ w_uk[h], k_rope] (width dn + dr) and its value is c_kv @ w_uv[h]
(width dv); the query is [q_nope, q_rope]; the score scale is 1/sqrt(dn + dr).

* ``mla_naive`` builds every head's keys and values from the latent and runs the plain
  attention definition (``oracle.attend``) with one KV head per query head.
* ``mla_absorbed`` never builds them: the query is moved into latent space
  (q_lat = q_nope @ w_uk[h]^T), scores are q_lat . c_kv + q_rope . k_rope, the softmax
  average is taken over the latents themselves, and w_uv is applied once per head to the
  averaged latent.  Over latents this is attention with a single shared KV head (keys
  [c_kv, k_rope], values c_kv), so it also runs through ``oracle.attend``.

The two are equal for any weights (the score identity q_nope . (c_kv @ w_uk) =
(q_nope @ w_uk^T) . c_kv, and the average commuting with the linear map w_uv); the pages
report 1.1e-15 on random weights.  Positions follow the same offset-causal rule as
``oracle.attend``: query row r of a Tq-row block at cache offset off_b sees tokens
j <= off_b + r.

Shapes: q_nope [B, H, Tq, dn], q_rope [B, H, Tq, dr], c_kv [B, Tcap, r],
k_rope [B, Tcap, dr], w_uk [H, r, dn], w_uv [H, r, dv].
"""
from __future__ import annotations

import math

import numpy as np

from .attend import _f64, attend


def mla_naive(q_nope, q_rope, c_kv, k_rope, w_uk, w_uv, cache_off=None, scale=None):
    qn, qr, C, R = _f64(q_nope), _f64(q_rope), _f64(c_kv), _f64(k_rope)
    Wk, Wv = _f64(w_uk), _f64(w_uv)
    B, H, Tq, dn = qn.shape
    Tcap, dr = C.shape[1], R.shape[2]
    scale = 1.0 / math.sqrt(dn + dr) if scale is None else scale
    # every head's keys and values, rebuilt from the latent: [B, H, Tcap, dn + dr], [B, H, Tcap, dv]
    K = np.concatenate([np.einsum("btr,hrn->bhtn", C, Wk),
                        np.broadcast_to(R[:, None], (B, H, Tcap, dr))], axis=-1)
    V = np.einsum("btr,hrv->bhtv", C, Wv)
    Q = np.concatenate([qn, qr], axis=-1)
    return attend(Q, K, V, cache_off=cache_off, scale=scale)


def mla_absorbed(q_nope, q_rope, c_kv, k_rope, w_uk, w_uv, cache_off=None, scale=None, return_latent=False):
    qn, qr, C, R = _f64(q_nope), _f64(q_rope), _f64(c_kv), _f64(k_rope)
    Wk, Wv = _f64(w_uk), _f64(w_uv)
    B, H, Tq, dn = qn.shape
    dr = R.shape[2]
    scale = 1.0 / math.sqrt(dn + dr) if scale is None else scale
    q_lat = np.einsum("bhtn,hrn->bhtr", qn, Wk)          # the query moved into latent space
    Q = np.concatenate([q_lat, qr], axis=-1)              # [B, H, Tq, r + dr]
    K = np.concatenate([C, R], axis=-1)[:, None]          # one shared "KV head": [B, 1, Tcap, r + dr]
    o_lat = attend(Q, K, C[:, None], cache_off=cache_off, scale=scale)  # average of latents [B, H, Tq, r]
    o = np.einsum("bhtr,hrv->bhtv", o_lat, Wv)            # expanded once per head
    return (o, o_lat, q_lat) if return_latent else o
