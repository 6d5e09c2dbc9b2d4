"""GPU parity of attn_dsa_decode (token top-k sparse attention with an indexer) against the
float64 oracle (oracle/dsa.py), through the C ABI.

The kept token set of every query token is the top k of the fp64 indexer scores (equal
scores: lower token index), on both sides: the kernel scores in fp32 with a bound on each
score's rounding, and decides every token that the bound leaves near the threshold on an fp64
score.  So kept lists must equal the oracle's exactly.  A row whose k-th and next distinct
fp64 scores lie within 1e-12 (relative) of each other would be flagged as a near tie that
fp64 rounding order could decide either way; none occurs in these cases.  Outputs: max-abs
2e-2 (bf16), every row."""
import numpy as np
import pytest
import torch

import synth
from oracle import attend
from oracle.dsa import indexer_scores, sparse_attend, topk_keep
from sparse_offset_causal_amd import AttnError, attn_decode, attn_dsa_decode
from tests.gpu_helpers import BF16_TOL, announce, dev, host64, max_abs, require_gpu

pytestmark = pytest.mark.gpu

REL_GAP = 1e-12  # far above fp64 rounding of the indexer sums, far below fp32 resolution


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run(x, topk, **kw):
    return attn_dsa_decode(dev(x.q), dev(x.k), dev(x.v), dev(x.qi), dev(x.ki), dev(x.wi), topk,
                           cache_off=dev(x.cache_off), sink=dev(x.sink), want_kept=True, **kw)


def threshold_gap(sc, k):
    """Relative distance from the k-th largest score to the closest different score."""
    srt = np.sort(sc)[::-1]
    if k >= len(srt):
        return np.inf
    tau = srt[k - 1]
    other = sc[sc != tau]
    return float(np.min(np.abs(other - tau)) / max(abs(tau), 1e-300)) if other.size else np.inf


def check(x, topk, batches=None, **kw):
    o, kl, kc = run(x, topk, **kw)
    bs = list(range(x.q.shape[0])) if batches is None else batches
    sl = torch.tensor(bs)
    ref, keep, scores = sparse_attend(x.q[sl], x.k[sl], x.v[sl], x.qi[sl], x.ki[sl], x.wi[sl], topk,
                                      cache_off=x.cache_off[sl], sink=x.sink, return_keep=True)
    kl, kc, o = kl.cpu().numpy(), kc.cpu().numpy(), host64(o)
    tq = x.q.shape[2]
    worst, gap = 0.0, np.inf
    for i, b in enumerate(bs):
        for t in range(tq):
            n_vis = int(x.cache_off[b]) + t + 1
            gap = min(gap, threshold_gap(scores[i, t, :n_vis], topk))
            want = np.nonzero(keep[i, t])[0]
            got = kl[b, t, :kc[b, t]]
            assert kc[b, t] == len(want), (b, t)
            assert np.array_equal(got, want), (b, t, np.setxor1d(got, want))
            worst = max(worst, max_abs(o[b, :, t], ref[i, :, t]))
    announce(f"  kept lists exact; smallest relative gap at a threshold {gap:.2e}; max-abs {worst:.2e}")
    assert gap > REL_GAP, "near tie: the kept set is not determined by fp64 evaluation"
    assert worst <= BF16_TOL, worst


@pytest.mark.parametrize("topk,split", [(16, 0), (100, 32), (64, 1000)])
def test_dsa_decode_matches_oracle(topk, split):
    announce(f"dsa decode topk={topk} split={split}")
    x = synth.dsa_inputs(B=4, Hq=8, Hkv=2, lengths=[0, 15, 300, 1200], Hi=16, seed=topk)
    check(x, topk, split_tokens=split)


@pytest.mark.parametrize("Hi,tq", [(64, 1), (32, 3), (48, 2)])
def test_dsa_decode_heads_and_query_tokens(Hi, tq):
    announce(f"dsa decode Hi={Hi} tq={tq}")
    x = synth.dsa_inputs(B=3, Hq=32, Hkv=8, tq=tq, lengths=[40, 500, 2000], Hi=Hi, seed=Hi + tq)
    check(x, 128)


def test_dsa_topk_covering_everything_is_dense():
    x = synth.dsa_inputs(B=3, Hq=8, Hkv=2, tq=2, lengths=[5, 77, 300], Hi=16, seed=9)
    o, kl, kc = run(x, 4096)
    dense = attn_decode(dev(x.q), dev(x.k), dev(x.v), cache_off=dev(x.cache_off), sink=dev(x.sink))
    assert torch.equal(kc.cpu(), (x.cache_off[:, None] + torch.arange(2)[None] + 1).to(torch.int32))
    assert max_abs(o, dense) <= 1e-2
    assert max_abs(o, attend(x.q, x.k, x.v, cache_off=x.cache_off, sink=x.sink)) <= BF16_TOL


def test_dsa_decode_full_size_B64_topk2048():
    announce("dsa decode full size")
    x = synth.dsa_inputs(B=64, Hq=32, Hkv=8, Hi=64, seed=0)
    L = x.cache_off.numpy()
    check(x, 2048, batches=sorted({0, 13, 37, 63, int(np.argmin(L)), int(np.argmax(L))}))


def test_dsa_decode_many_short_rows_per_workgroup():
    """2048 short rows (64 sequences x 32 query tokens, 100-300 cached tokens): each indexer
    workgroup's share of the blocks spans about eight rows, more than one phase stages, so
    shares are cut into several phases, and row windows past the first 64 rows are read."""
    announce("dsa decode 64 x 32 short rows")
    x = synth.dsa_inputs(B=64, Hq=8, Hkv=8, tq=32, lo=100, hi=300, Hi=16, seed=31)
    check(x, 64, batches=[0, 21, 63])


def test_dsa_decode_long_rows_multi_phase():
    """8 sequences of 300k-320k cached tokens: each indexer workgroup's share exceeds the
    blocks one phase holds, so a row's blocks are split over phases (and over workgroups)."""
    announce("dsa decode 8 x ~310k tokens")
    x = synth.dsa_inputs(B=8, Hq=8, Hkv=1, lo=300000, hi=320000, Hi=16, seed=32)
    check(x, 256, batches=[0, 5])


def test_dsa_decode_rejects_bad_index_heads():
    x = synth.dsa_inputs(B=1, Hq=8, Hkv=2, lengths=[10], Hi=8, seed=1)
    with pytest.raises(AttnError, match="index_heads"):
        run(x, 4)


def tie_row_for(x, scale=4.0):
    """A key row along the positively weighted indexer queries: it scores far above random rows."""
    w, qv = x.wi[0, :, 0].float(), x.qi[0, :, 0].float()
    dirn = (w.clamp(min=0)[:, None] * qv).sum(0)
    return (dirn / dirn.norm() * scale * 128 ** 0.5).to(x.ki.dtype)


@pytest.mark.parametrize("n_tied,extra", [(600, 250), (3000, 1700)])
def test_dsa_topk_exact_ties_keep_lowest_indices(n_tied, extra):
    """n_tied tokens share one indexer key row (bitwise-equal scores on both sides); 30 tokens
    carry twice that row (strictly larger scores).  top-k then cuts inside the tie group, and
    the kept set must be the larger tokens plus the lowest-indexed tied ones, exactly; the tie
    group spans the token segments of several waves of the selection kernel, and the larger
    case holds more tied tokens than there are threads in its workgroup."""
    announce(f"dsa top-k exact ties n_tied={n_tied}")
    x = synth.dsa_inputs(B=1, Hq=8, Hkv=2, lengths=[10000], Hi=16, seed=21)
    tie_row = tie_row_for(x)
    tie_score = indexer_scores(x.qi, tie_row.view(1, 1, -1), x.wi)[0, 0, 0]
    assert tie_score > 0
    tied = torch.arange(200, 200 + 3 * n_tied, 3)
    top = torch.arange(9500, 9530)
    x.ki[0, tied] = tie_row
    x.ki[0, top] = (tie_row.float() * 2).to(x.ki.dtype)  # exact in bf16
    scores = indexer_scores(x.qi, x.ki, x.wi)[0, 0, :10001]
    n_gt = int((scores > tie_score).sum())
    assert int((scores == tie_score).sum()) == n_tied and n_gt == 30
    topk = n_gt + extra
    keep = topk_keep(indexer_scores(x.qi, x.ki, x.wi), topk, x.cache_off)
    want = np.nonzero(keep[0, 0])[0]
    assert np.array_equal(want[np.isin(want, tied.numpy())], tied.numpy()[:extra])
    o, kl, kc = run(x, topk)
    got = kl.cpu().numpy()[0, 0, :int(kc[0, 0])]
    assert np.array_equal(got, want)
    ref = sparse_attend(x.q, x.k, x.v, x.qi, x.ki, x.wi, topk, cache_off=x.cache_off, sink=x.sink)
    assert max_abs(o, ref) <= BF16_TOL


def test_dsa_topk_decided_below_fp32_resolution():
    """400 tokens carry one high-scoring key row in which 100 dimensions are zero; each token
    then holds one tiny value (+-2^-18 .. 2^-21) in one of those dimensions.  Their fp64 scores
    all differ, by about 1e-7 of the score or less, below what fp32 indexer scores resolve.
    top-k cuts inside this group, so only an fp64 decision reproduces the oracle's kept set."""
    announce("dsa top-k below fp32 resolution")
    x = synth.dsa_inputs(B=1, Hq=8, Hkv=2, lengths=[6000], Hi=32, seed=23)
    g = torch.Generator().manual_seed(24)
    base = tie_row_for(x).float()
    dims = torch.randperm(128, generator=g)[:100]
    base[dims] = 0.0
    toks = torch.arange(1000, 1000 + 400 * 7, 7)
    rows = base.repeat(len(toks), 1)
    for n in range(len(toks)):
        rows[n, int(dims[n % 100])] = (1.0 if n % 2 else -1.0) * 2.0 ** -(18 + n // 100)
    x.ki[0, toks] = rows.to(x.ki.dtype)
    assert torch.equal(x.ki[0, toks].float(), rows)  # every value exact in bf16
    sc = indexer_scores(x.qi, x.ki, x.wi)[0, 0, :6001]
    grp = sc[toks.numpy()]
    assert len(np.unique(grp)) == len(toks)
    assert (grp.max() - grp.min()) / grp.max() < 1e-6
    topk = int((sc > grp.max()).sum()) + 200
    check(x, topk)
