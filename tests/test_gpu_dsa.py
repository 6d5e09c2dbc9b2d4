"""GPU parity of attn_dsa_decode (token top-k sparse attention with an indexer) against the
float64 oracle (oracle/dsa.py), through the C ABI.

The kept token sets are compared exactly.  The kernel computes indexer scores in fp32 from
bf16 inputs, the oracle in fp64; a token may only differ between the two sets if its score
lies within fp32 rounding of the threshold (a near tie) - the test checks that and then
skips that row's output comparison.  Outputs: max-abs 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

import synth
from oracle import attend
from oracle.dsa import indexer_scores, sparse_attend, topk_keep
from sparse_offset_causal_amd import AttnError, attn_decode, attn_dsa_decode
from tests.gpu_helpers import BF16_TOL, announce, dev, host64, max_abs, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run(x, topk, **kw):
    return attn_dsa_decode(dev(x.q), dev(x.k), dev(x.v), dev(x.qi), dev(x.ki), dev(x.wi), topk,
                           cache_off=dev(x.cache_off), sink=dev(x.sink), want_kept=True, **kw)


def check(x, topk, batches=None, **kw):
    o, kl, kc = run(x, topk, **kw)
    bs = list(range(x.q.shape[0])) if batches is None else batches
    sl = torch.tensor(bs)
    ref, keep, scores = sparse_attend(x.q[sl], x.k[sl], x.v[sl], x.qi[sl], x.ki[sl], x.wi[sl], topk,
                                      cache_off=x.cache_off[sl], sink=x.sink, return_keep=True)
    kl, kc, o = kl.cpu().numpy(), kc.cpu().numpy(), host64(o)
    worst, near = 0.0, 0
    tq = x.q.shape[2]
    for i, b in enumerate(bs):
        for t in range(tq):
            want = np.nonzero(keep[i, t])[0]
            got = np.sort(kl[b, t, :kc[b, t]])
            assert kc[b, t] == len(want)
            assert np.array_equal(got, kl[b, t, :kc[b, t]]), "list not ascending"
            if not np.array_equal(got, want):
                diff = np.setxor1d(got, want)
                sc = scores[i, t]
                tau = np.sort(sc[: int(x.cache_off[b]) + t + 1])[::-1][topk - 1]
                assert np.all(np.abs(sc[diff] - tau) <= 1e-5 * np.max(np.abs(sc))), (b, t, diff)
                near += 1
                continue
            worst = max(worst, max_abs(o[b, :, t], ref[i, :, t]))
    assert worst <= BF16_TOL, worst
    return near


@pytest.mark.parametrize("topk,split", [(16, 0), (100, 32), (64, 1000)])
def test_dsa_decode_matches_oracle(topk, split):
    announce(f"dsa decode topk={topk} split={split}")
    x = synth.dsa_inputs(B=4, Hq=8, Hkv=2, lengths=[0, 15, 300, 1200], Hi=16, seed=topk)
    assert check(x, topk, split_tokens=split) == 0


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
    near = check(x, 2048, batches=[0, 13, 37, 63])
    assert near <= 1


def test_dsa_decode_rejects_bad_index_heads():
    x = synth.dsa_inputs(B=1, Hq=8, Hkv=2, lengths=[10], Hi=8, seed=1)
    with pytest.raises(AttnError, match="index_heads"):
        run(x, 4)


def test_dsa_topk_exact_ties_keep_lowest_indices():
    """600 tokens share one indexer key row (bitwise-equal scores on both sides); 30 tokens
    carry twice that row (strictly larger scores).  top-k then cuts inside the tie group, and
    the kept set must be the larger tokens plus the lowest-indexed tied ones, exactly; the tie
    group spans the token segments of several waves of the selection kernel."""
    announce("dsa top-k exact ties")
    x = synth.dsa_inputs(B=1, Hq=8, Hkv=2, lengths=[5000], Hi=16, seed=21)
    # a key row along the positively weighted indexer queries scores far above random rows
    w, qv = x.wi[0, :, 0].float(), x.qi[0, :, 0].float()
    dirn = (w.clamp(min=0)[:, None] * qv).sum(0)
    tie_row = (dirn / dirn.norm() * 4 * 128 ** 0.5).to(x.ki.dtype)
    tie_score = indexer_scores(x.qi, tie_row.view(1, 1, -1), x.wi)[0, 0, 0]
    assert tie_score > 0
    tied = torch.arange(200, 200 + 3 * 600, 3)
    top = torch.arange(2500, 2530)
    x.ki[0, tied] = tie_row
    x.ki[0, top] = (tie_row.float() * 2).to(x.ki.dtype)  # exact in bf16
    scores = indexer_scores(x.qi, x.ki, x.wi)[0, 0, :5001]
    n_gt = int((scores > tie_score).sum())
    assert int((scores == tie_score).sum()) == 600 and n_gt == 30
    topk = n_gt + 250
    keep = topk_keep(indexer_scores(x.qi, x.ki, x.wi), topk, x.cache_off)
    want = np.nonzero(keep[0, 0])[0]
    assert np.array_equal(want[np.isin(want, tied.numpy())], tied.numpy()[:250])
    o, kl, kc = run(x, topk)
    got = kl.cpu().numpy()[0, 0, :int(kc[0, 0])]
    assert np.array_equal(got, want)
    ref = sparse_attend(x.q, x.k, x.v, x.qi, x.ki, x.wi, topk, cache_off=x.cache_off, sink=x.sink)
    assert max_abs(o, ref) <= BF16_TOL
