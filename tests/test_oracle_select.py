"""Pins for the block-selection oracle (CPU only).

Ties oracle.select to: an independent scalar brute force (explicit loops over
every row and key), exact keep counts, monotonicity in the keep fractions, the
closed-form count of admissible block pairs, recovery of planted outlier keys
that the mean-centroid score dilutes (patty.io RBS-Attention review, sections on
mean dilution and the radius rescue), and "keep everything equals dense".
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import attend, block_list_from_mask, select_blocks
from oracle.brute import select_brute
from oracle.select import admissible


def _qk(B, Hq, Hkv, Tq, Tcap, d, seed):
    w = synth.attention_inputs(B, Hq, Hkv, Tq, Tcap, d, torch.bfloat16, seed)
    return w.q, w.k


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Tq, Tcap, bs, offsets, window
    (1, 4, 2, 24, 24, 4, None, 0),
    (1, 2, 1, 21, 21, 4, None, 0),      # short last blocks
    (2, 4, 2, 10, 25, 4, [15, 3], 0),   # per-sequence cache offsets
    (1, 4, 2, 24, 24, 4, None, 7),      # window
    (1, 2, 2, 9, 30, 3, [21], 5),
])
@pytest.mark.parametrize("keeps", [(0.05, 0.05), (0.3, 0.0), (0.0, 0.4), (0.5, 0.5), (1.0, 0.0)])
def test_select_matches_brute_force(case, keeps):
    B, Hq, Hkv, Tq, Tcap, bs, offs, W = case
    q, k = _qk(B, Hq, Hkv, Tq, Tcap, 8, seed=21)
    sel = select_blocks(q, k, bs, cache_off=offs, window=W, keep_mean=keeps[0], keep_radius=keeps[1])
    mask_b, t1, t2 = select_brute(q, k, bs, cache_off=offs, window=W, keep_mean=keeps[0],
                                  keep_radius=keeps[1])
    assert np.array_equal(sel["mask"], np.array(mask_b, dtype=np.uint8))
    np.testing.assert_allclose(sel["tau_mean"], t1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sel["tau_radius"], t2, rtol=1e-12, atol=1e-14)


def test_admissible_matches_rule_by_enumeration():
    rng = np.random.default_rng(0)
    for _ in range(40):
        bs = int(rng.integers(1, 6))
        tq = int(rng.integers(1, 30))
        off = int(rng.integers(0, 20))
        W = int(rng.integers(0, 12))
        tkb = off + tq
        adm = admissible(tq, tkb, off, W, bs)
        for qb in range(adm.shape[0]):
            for kb in range(adm.shape[1]):
                want = any(j <= off + r and (W <= 0 or j > off + r - W)
                           for r in range(qb * bs, min((qb + 1) * bs, tq))
                           for j in range(kb * bs, min((kb + 1) * bs, tkb)))
                assert adm[qb, kb] == want


def test_admissible_pair_count_closed_form():
    nb = 512
    assert admissible(nb * 128, nb * 128, 0, 0, 128).sum() == nb * (nb + 1) // 2 == 131328


def test_exact_keep_counts_without_ties():
    q, k = _qk(1, 4, 2, 64 * 8, 64 * 8, 16, seed=3)
    for frac in (0.05, 0.1, 0.37):
        sel = select_blocks(q, k, 8, keep_mean=frac, keep_radius=0.0)
        n_adm = sel["adm"][0].sum()
        for h in range(4):
            assert sel["mask"][0, h].sum() == math.floor(frac * n_adm + 0.5)
        sel = select_blocks(q, k, 8, keep_mean=0.0, keep_radius=frac)
        for h in range(4):
            cols = sel["mask"][0, h].any(axis=0).sum()
            assert cols == math.floor(frac * 64 + 0.5)


def test_selection_is_monotone_in_keep_fractions():
    q, k = _qk(1, 4, 2, 40 * 6, 40 * 6, 16, seed=4)
    prev = None
    for frac in (0.0, 0.02, 0.05, 0.1, 0.3, 1.0):
        m = select_blocks(q, k, 6, keep_mean=frac, keep_radius=frac / 2)["mask"].astype(bool)
        if prev is not None:
            assert np.all(m >= prev)
        prev = m


def test_keep_all_selects_every_admissible_pair_and_equals_dense():
    q, k = _qk(1, 4, 2, 30, 30, 8, seed=5)
    v = synth.normal((1, 2, 30, 8), 99, torch.bfloat16)
    sel = select_blocks(q, k, 4, keep_mean=1.0, keep_radius=0.0)
    assert np.array_equal(sel["mask"][0].astype(bool), np.broadcast_to(sel["adm"][0], (4,) + sel["adm"][0].shape))
    dense = attend(q, k, v)
    sparse = attend(q, k, v, block_mask=sel["mask"], block_size=4)
    assert np.array_equal(dense, sparse)


def test_absolute_threshold_mode():
    q, k = _qk(1, 4, 2, 48, 48, 16, seed=6)
    sel = select_blocks(q, k, 8, keep_mean=0.2, keep_radius=0.1)
    again = select_blocks(q, k, 8, keep_mean=-1.0, keep_radius=-1.0,
                          tau_mean=sel["tau_mean"], tau_radius=sel["tau_radius"])
    assert np.array_equal(sel["mask"], again["mask"])


def test_planted_outliers_recovered_by_radius_branch():
    # 32 key blocks per head, 4 planted (frac 1/8).  The radius branch alone with the
    # matching keep fraction selects exactly the planted key-block columns.
    w = synth.block_sparse_prefill(T=4096, BS=128, Hq=8, Hkv=2, d=64, frac=0.125)
    planted = {(kvh, kb) for kvh, kb, _, _ in w.meta["planted"]}
    sel = select_blocks(w.q, w.k, 128, keep_mean=0.0, keep_radius=0.125)
    for kvh in range(2):
        top = set(np.argsort(-sel["rad2"][0, kvh])[:4].tolist())
        assert top == {kb for (kv, kb) in planted if kv == kvh}
        assert np.all((sel["rad2"][0, kvh] > sel["tau_radius"][0, kvh]) ==
                      np.isin(np.arange(32), sorted(top)))
        for h in range(kvh * 4, kvh * 4 + 4):
            cols = set(np.nonzero(sel["mask"][0, h].any(axis=0))[0].tolist())
            assert cols == top
    # the mean branch at the same budget misses some planted blocks (mean dilution)
    mean_only = select_blocks(w.q, w.k, 128, keep_mean=4 / 528, keep_radius=0.0)["mask"]
    hits = sum(mean_only[0, h][:, kb].any() for (kvh, kb) in planted for h in range(kvh * 4, kvh * 4 + 4))
    assert hits < 4 * len(planted)


def test_block_list_from_mask():
    m = np.array([[[[1, 0, 1, 1], [0, 0, 0, 0]]]], dtype=np.uint8)
    lst = block_list_from_mask(m)
    assert lst.tolist() == [[[[3, 0, 2, 3, 0], [0, 0, 0, 0, 0]]]]
