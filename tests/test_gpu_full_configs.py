"""Parity at the benchmark workloads' full sizes, in the launch configuration bench.py times.

The GPU computes every output; the float64 oracle recomputes sampled rows (tile edges,
first/last rows, random rows) of sampled heads, and every output element is checked to be
finite.  The block-sparse workload's mask is compared bit-exactly over all heads.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attend, select_blocks
from sparse_offset_causal_amd import attn_block_select, attn_block_sparse_prefill, attn_decode, attn_prefill
from tests.gpu_helpers import BF16_TOL, announce, host64, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def sample_rows(T, n_random=24, seed=0):
    edges = [0, 1, 63, 64, 127, 128, 129, T // 2 - 1, T // 2, T - 129, T - 128, T - 2, T - 1]
    rnd = np.random.default_rng(seed).integers(0, T, n_random).tolist()
    return sorted({r for r in edges + rnd if 0 <= r < T})


def check_rows(o, w, rows, heads, **kw):
    ref = attend(w.q, w.k, w.v, cache_off=w.cache_off, window=w.window, sink=w.sink, scale=w.scale, rows=rows,
                 heads=heads, **kw)
    got = host64(o[:, heads][:, :, rows])
    err = float(np.max(np.abs(got - ref)))
    announce(f"{w.name}: sampled max-abs err {err:.3e} over {len(rows)} rows x {len(heads)} heads")
    assert err <= BF16_TOL
    assert bool(torch.isfinite(o).all())


def test_causal_prefill_T8192_full_size():
    w = synth.causal_prefill(T=8192)
    o = attn_prefill(w.q.cuda(), w.k.cuda(), w.v.cuda(), cache_off=w.cache_off.cuda(), scale=w.scale)
    check_rows(o, w, sample_rows(8192), [0, 3, 17, 31])


def test_window_sink_prefill_T32768_full_size():
    w = synth.window_sink_prefill(T=32768, W=1024)
    o = attn_prefill(w.q.cuda(), w.k.cuda(), w.v.cuda(), cache_off=w.cache_off.cuda(), window=1024,
                     sink=w.sink.cuda())
    # every head: the workgroups stack 4 heads of a KV group, so each head position in the stack
    # and each KV group is covered
    check_rows(o, w, sample_rows(32768, 12), list(range(32)))


def test_decode_and_chunk_B64_full_size():
    c = synth.decode_cache(B=64)
    k, v, off = c.k.cuda(), c.v.cuda(), c.lengths.cuda()
    od = attn_decode(c.q_decode.cuda(), k, v, cache_off=off)
    wd = c.decode()
    heads = [0, 7, 8, 31]
    ref = attend(wd.q, wd.k, wd.v, cache_off=wd.cache_off, heads=heads)
    err = float(np.max(np.abs(host64(od[:, heads]) - ref)))
    announce(f"decode B=64: max-abs err {err:.3e} over all 64 sequences x {len(heads)} heads")
    assert err <= BF16_TOL and bool(torch.isfinite(od).all())
    oc = attn_prefill(c.q_chunk.cuda(), k, v, cache_off=off)
    wc = c.prefill_chunk()
    # all 32 heads of 8 sequences (the shortest and longest caches among them) at the rows on
    # either side of every 32-row wave block and 128-row workgroup edge
    rows = [0, 1, 31, 32, 63, 64, 95, 96, 127, 128, 255, 256, 383, 384, 510, 511]
    L = c.lengths.numpy()
    seqs = sorted({int(np.argmin(L)), int(np.argmax(L)), 0, 9, 17, 30, 45, 63})
    ref = attend(wc.q, wc.k, wc.v, cache_off=wc.cache_off, rows=rows, batches=seqs)
    err = float(np.max(np.abs(host64(oc[seqs][:, :, rows]) - ref)))
    announce(f"chunk 512 at cache offsets: max-abs err {err:.3e} over {len(seqs)} sequences x 32 heads x "
             f"{len(rows)} rows")
    assert err <= BF16_TOL and bool(torch.isfinite(oc).all())


def test_block_sparse_T65536_full_size():
    w = synth.block_sparse_prefill(T=65536, BS=128)
    q, k, v = w.q.cuda(), w.k.cuda(), w.v.cuda()
    sel = attn_block_select(q, k, block_size=128, keep_mean=w.keep_mean, keep_radius=w.keep_radius)
    announce("block select done on GPU; running the oracle selection for all 32 heads")
    ref = select_blocks(w.q, w.k, 128, keep_mean=w.keep_mean, keep_radius=w.keep_radius)
    mask = sel["mask"].cpu().numpy()
    assert np.array_equal(mask, ref["mask"])
    kept = mask.sum() / (32 * 512 * 513 / 2)
    announce(f"block mask bit-exact over 32 heads; kept fraction {kept:.4f}")
    assert 0.07 < kept < 0.13
    # the radius branch keeps every planted key block (its column, in every head of the group)
    for kvh, kb, _, qb in w.meta["planted"]:
        assert mask[0, 4 * kvh:4 * kvh + 4, kb:, kb].all()
    o = attn_prefill(q, k, v, block_list=sel["list"], block_size=128)
    check_rows(o, w, sample_rows(65536, 16), [2, 29], block_mask=ref["mask"], block_size=128)


def test_chunk_block_sparse_B64_full_size():
    """The 512-token chunk at every sequence's cache offset (batch 64, cache lengths in [1024,
    32768]) with query-chunked block selection fused into the prefill: the selection's mask is
    bit-exact against the oracle's for sampled sequences (their whole K cache at each offset), and
    sampled rows of every head match the oracle's attention over that mask."""
    c = synth.decode_cache(B=64)
    k, v, off = c.k.cuda(), c.v.cuda(), c.lengths.cuda()
    q = c.q_chunk.cuda()
    o, sel = attn_block_sparse_prefill(q, k, v, cache_off=off, keep_mean=0.05, keep_radius=0.05, want_mask=True)
    mask = sel["mask"].cpu().numpy()
    L = c.lengths.numpy()
    seqs = sorted({int(np.argmin(L)), int(np.argmax(L)), 5, 40})
    rows = [0, 1, 127, 128, 255, 256, 383, 384, 511]
    worst = 0.0
    for bq in seqs:
        sl = slice(bq, bq + 1)
        ref_sel = select_blocks(c.q_chunk[sl], c.k[sl], 128, cache_off=[int(L[bq])], keep_mean=0.05, keep_radius=0.05)
        assert np.array_equal(mask[sl], ref_sel["mask"]), bq
        ref = attend(c.q_chunk[sl], c.k[sl], c.v[sl], cache_off=[int(L[bq])], rows=rows, block_mask=ref_sel["mask"],
                     block_size=128)
        worst = max(worst, float(np.max(np.abs(host64(o[sl][:, :, rows]) - ref))))
    kept = mask.sum() / max(1, int(sum(4 * (int(l) // 128 + 1) for l in L)) * 32)
    announce(f"chunk block-sparse: masks bit-exact for {len(seqs)} sequences, max-abs {worst:.3e}, kept ~{kept:.3f}")
    assert worst <= BF16_TOL and bool(torch.isfinite(o).all())
