"""Pins of the MLA oracle (oracle/mla.py) to things other than itself (sotaaz.com/post/
attention-in-code, section 4).

* naive == absorbed for random weights: an identity of the mathematics (the pages report
  1.1e-15); a mistake in either form (a dropped transpose, the rope part missing, w_uv
  applied to the wrong side) breaks it;
* a two-token case worked out by hand with math.exp;
* identity weights and no rope part reduce MLA to plain attention with one shared KV head,
  checked against the scalar brute force;
* the default score scale is 1/sqrt(dn + dr) (not 1/sqrt(dn));
* decode one token at a time at offsets 0..T-1 equals the one-shot computation.
"""
import math

import numpy as np
import pytest

from oracle.brute import attend_brute
from oracle.mla import mla_absorbed, mla_naive


def rand_mla(B=2, H=4, Tq=3, T=20, dn=16, dr=8, r=32, dv=16, seed=0):
    rng = np.random.default_rng(seed)
    return dict(q_nope=rng.standard_normal((B, H, Tq, dn)), q_rope=rng.standard_normal((B, H, Tq, dr)),
                c_kv=rng.standard_normal((B, T, r)), k_rope=rng.standard_normal((B, T, dr)),
                w_uk=rng.standard_normal((H, r, dn)) / math.sqrt(r), w_uv=rng.standard_normal((H, r, dv)) / math.sqrt(r))


@pytest.mark.parametrize("offs", [None, [0, 17], [5, 9]])
def test_naive_equals_absorbed(offs):
    x = rand_mla()
    a = mla_naive(**x, cache_off=offs)
    b = mla_absorbed(**x, cache_off=offs)
    assert np.max(np.abs(a - b)) < 1e-13


def test_naive_equals_absorbed_decode_many_heads():
    x = rand_mla(B=3, H=16, Tq=1, T=70, dn=32, dr=16, r=64, dv=24, seed=4)
    a = mla_naive(**x, cache_off=[0, 33, 69])
    b = mla_absorbed(**x, cache_off=[0, 33, 69])
    assert np.max(np.abs(a - b)) < 1e-13


def test_two_token_closed_form():
    # H = 1, widths 1: scores s_j = (a*u*c_j + b*r_j) / sqrt(2); o = w * (p0 c0 + p1 c1)
    a, b, u, w = 0.7, -1.3, 1.9, 0.6
    c = [0.4, -2.1]
    rr = [1.5, 0.2]
    x = dict(q_nope=np.array(a).reshape(1, 1, 1, 1), q_rope=np.array(b).reshape(1, 1, 1, 1),
             c_kv=np.array(c).reshape(1, 2, 1), k_rope=np.array(rr).reshape(1, 2, 1),
             w_uk=np.array(u).reshape(1, 1, 1), w_uv=np.array(w).reshape(1, 1, 1))
    s = [(a * u * c[j] + b * rr[j]) / math.sqrt(2.0) for j in range(2)]
    e = [math.exp(v - max(s)) for v in s]
    want = w * (e[0] * c[0] + e[1] * c[1]) / (e[0] + e[1])
    for f in (mla_naive, mla_absorbed):
        assert abs(float(f(**x, cache_off=[1])[0, 0, 0, 0]) - want) < 1e-15
    # at offset 0 the query sees token 0 only
    for f in (mla_naive, mla_absorbed):
        assert abs(float(f(**x, cache_off=[0])[0, 0, 0, 0]) - w * c[0]) < 1e-15


def test_identity_weights_reduce_to_shared_head_attention():
    rng = np.random.default_rng(7)
    B, H, Tq, T, d = 1, 3, 4, 9, 5
    qn = rng.standard_normal((B, H, Tq, d))
    C = rng.standard_normal((B, T, d))
    eye = np.broadcast_to(np.eye(d), (H, d, d)).copy()
    empty_q, empty_k = np.zeros((B, H, Tq, 0)), np.zeros((B, T, 0))
    got = mla_absorbed(qn, empty_q, C, empty_k, eye, eye, cache_off=[5])
    got_n = mla_naive(qn, empty_q, C, empty_k, eye, eye, cache_off=[5])
    ref = np.array(attend_brute(qn, C[:, None], C[:, None], cache_off=[5]))
    assert np.max(np.abs(got - ref)) < 1e-13 and np.max(np.abs(got_n - ref)) < 1e-13


def test_default_scale_counts_the_rope_width():
    x = rand_mla(seed=2)
    dn, dr = 16, 8
    a = mla_absorbed(**x)
    assert np.max(np.abs(a - mla_absorbed(**x, scale=1 / math.sqrt(dn + dr)))) == 0.0
    assert np.max(np.abs(a - mla_absorbed(**x, scale=1 / math.sqrt(dn)))) > 1e-3


def test_decode_token_by_token_equals_one_shot():
    x = rand_mla(B=1, H=2, Tq=12, T=12, seed=3)
    full = mla_absorbed(**x, cache_off=[0])
    for t in range(12):
        step = dict(x, q_nope=x["q_nope"][:, :, t:t + 1], q_rope=x["q_rope"][:, :, t:t + 1])
        assert np.max(np.abs(mla_absorbed(**step, cache_off=[t])[:, :, 0] - full[:, :, t])) < 1e-13
