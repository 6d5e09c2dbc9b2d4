"""Pins of the sparse-attention oracle (oracle/dsa.py) to things other than itself
(sotaaz.com/post/attention-in-code, section 5).

* k at least the visible count gives dense attention exactly (difference 0, as the pages
  report);
* the indexer score against a scalar loop, and a negative check that the ReLU matters;
* kept counts: min(k, visible) per query token (the pages' 60-token, k = 16 example: the
  last query reads 16 tokens);
* the kept set against a brute-force sort, including exact ties (ReLU zeros), which go to
  the lower token index;
* attention over the kept set equals the scalar brute force with the same mask.
"""
import math

import numpy as np
import pytest

from oracle import attend
from oracle.brute import attend_brute
from oracle.dsa import indexer_scores, sparse_attend, topk_keep


def rand_dsa(B=2, Hq=4, Hkv=2, Tq=3, T=60, d=16, Hi=3, di=8, seed=0):
    rng = np.random.default_rng(seed)
    return dict(q=rng.standard_normal((B, Hq, Tq, d)), k=rng.standard_normal((B, Hkv, T, d)),
                v=rng.standard_normal((B, Hkv, T, d)), qi=rng.standard_normal((B, Hi, Tq, di)),
                ki=rng.standard_normal((B, T, di)), wi=rng.standard_normal((B, Hi, Tq)))


@pytest.mark.parametrize("offs", [None, [10, 57]])
def test_k_at_least_visible_is_dense_exactly(offs):
    x = rand_dsa()
    o = sparse_attend(**x, topk=60, cache_off=offs)
    dense = attend(x["q"], x["k"], x["v"], cache_off=offs)
    assert np.array_equal(o, dense)


def test_indexer_scores_match_scalar_loop():
    x = rand_dsa(B=1, Tq=2, T=7, Hi=3, di=4, seed=1)
    S = indexer_scores(x["qi"], x["ki"], x["wi"])
    for t in range(2):
        for s in range(7):
            want = 0.0
            for j in range(3):
                dot = sum(x["qi"][0, j, t, e] * x["ki"][0, s, e] for e in range(4))
                want += x["wi"][0, j, t] * max(dot, 0.0)
            assert abs(S[0, t, s] - want) < 1e-13
    no_relu = np.einsum("bjt,bjts->bts", x["wi"], np.einsum("bjtd,bsd->bjts", x["qi"], x["ki"]))
    assert np.max(np.abs(S - no_relu)) > 1e-3


def test_kept_counts_follow_min_k_visible():
    x = rand_dsa(B=1, Tq=60, T=60, seed=2)
    keep = topk_keep(indexer_scores(x["qi"], x["ki"], x["wi"]), 16, cache_off=[0])
    counts = keep.sum(-1)[0]
    assert counts[-1] == 16
    assert list(counts) == [min(16, t + 1) for t in range(60)]
    # never a token beyond the query's position
    for t in range(60):
        assert not keep[0, t, t + 1:].any()


def test_kept_set_brute_force_with_exact_ties():
    rng = np.random.default_rng(3)
    scores = np.round(rng.standard_normal((1, 4, 30)), 1)  # many exact ties
    scores[0, :, ::3] = 0.0                                  # ReLU-style zeros
    keep = topk_keep(scores, 9, cache_off=[26])
    for t in range(4):
        n_vis = 26 + t + 1
        items = sorted(range(n_vis), key=lambda s: (-scores[0, t, s], s))
        assert set(np.nonzero(keep[0, t])[0].tolist()) == set(items[:9])


def test_sparse_output_matches_brute_force_with_same_mask():
    x = rand_dsa(B=1, Hq=4, Hkv=2, Tq=2, T=12, d=5, seed=4)
    o, keep, _ = sparse_attend(**x, topk=4, cache_off=[10], return_keep=True)
    mask = np.broadcast_to(keep[:, None], (1, 4) + keep.shape[1:])
    ref = np.array(attend_brute(x["q"], x["k"], x["v"], cache_off=[10], block_mask=mask, block_size=1))
    assert np.max(np.abs(o - ref)) < 1e-13
    assert np.max(np.abs(o - attend(x["q"], x["k"], x["v"], cache_off=[10]))) > 1e-3  # sparsity changes it
