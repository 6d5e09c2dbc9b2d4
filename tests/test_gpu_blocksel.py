"""GPU block selection against the float64 oracle: masks and kept lists bit-exact,
thresholds to float64 rounding, plus block-sparse prefill parity on the selected blocks.

Both sides compute in float64 from the same exactly widened inputs, so a decision can
only differ if a score lies within float64 rounding of its threshold; every case reports
the smallest relative gap and such a case would be flagged as a near tie, not accepted.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attend, block_list_from_mask, select_blocks
from sparse_offset_causal_amd import (attn_block_list_from_mask, attn_block_select, attn_block_sparse_prefill,
                                      attn_prefill)
from tests.gpu_helpers import BF16_TOL, announce, dev, host64, max_abs, require_gpu

pytestmark = pytest.mark.gpu

REL_EPS = 1e-12  # far above float64 rounding of a 128-term dot product, far below data gaps


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def min_gap(ref):
    """Smallest |value - tau| / |tau| over the values of both branches other than tau itself (the
    element that defines tau is dropped on both sides by the strict comparison)."""
    gaps = []
    s, t1 = ref["score"], ref["tau_mean"]
    for b in range(s.shape[0]):
        for h in range(s.shape[1]):
            if np.isfinite(t1[b, h]):
                v = s[b, h][np.isfinite(s[b, h]) & (s[b, h] != t1[b, h])]
                if v.size:
                    gaps.append(np.min(np.abs(v - t1[b, h])) / max(abs(t1[b, h]), 1e-300))
    r2, t2 = ref["rad2"], ref["tau_radius"]
    for b in range(r2.shape[0]):
        for kv in range(r2.shape[1]):
            if np.isfinite(t2[b, kv]):
                v = r2[b, kv][np.isfinite(r2[b, kv]) & (r2[b, kv] != t2[b, kv])]
                if v.size:
                    gaps.append(np.min(np.abs(v - t2[b, kv])) / max(abs(t2[b, kv]), 1e-300))
    return min(gaps) if gaps else np.inf


def lists_match(got_list, ref_mask):
    """Counts and kept entries equal (entries past each count are unspecified)."""
    ref = block_list_from_mask(ref_mask)
    got = got_list.cpu().numpy() if hasattr(got_list, "cpu") else got_list
    if not np.array_equal(got[..., 0], ref[..., 0]):
        return False
    for idx in np.ndindex(*ref.shape[:-1]):
        n = ref[idx][0]
        if not np.array_equal(got[idx][1:1 + n], ref[idx][1:1 + n]):
            return False
    return True


def check_select(q, k, bs, cache_off=None, window=0, keep_mean=0.05, keep_radius=0.05):
    ref = select_blocks(q, k, bs, cache_off=cache_off, window=window, keep_mean=keep_mean, keep_radius=keep_radius)
    off_t = None if cache_off is None else torch.tensor(cache_off, dtype=torch.int32, device="cuda")
    got = attn_block_select(dev(q), dev(k), block_size=bs, cache_off=off_t, window=window, keep_mean=keep_mean,
                            keep_radius=keep_radius)
    gap = min_gap(ref)
    announce(f"select bs={bs} window={window} keeps=({keep_mean},{keep_radius}) min relative gap {gap:.3e}")
    assert gap > REL_EPS, "near tie: decision not determined by float64 evaluation"
    assert np.array_equal(got["mask"].cpu().numpy(), ref["mask"])
    assert lists_match(got["list"], ref["mask"])
    np.testing.assert_allclose(host64(got["tau_mean"]), ref["tau_mean"], rtol=REL_EPS)
    np.testing.assert_allclose(host64(got["tau_radius"]), ref["tau_radius"], rtol=REL_EPS)
    return ref, got


def test_select_planted_outliers_bit_exact():
    w = synth.block_sparse_prefill(T=2048, BS=128, Hq=8, Hkv=2, d=128, frac=0.125, keep_mean=0.05,
                                   keep_radius=0.125)
    ref, got = check_select(w.q, w.k, 128, keep_mean=0.05, keep_radius=0.125)
    planted = {(kvh, kb) for kvh, kb, _, _ in w.meta["planted"]}
    # the radius branch rescues exactly the planted key blocks (columns of every head in the group)
    mask = got["mask"].cpu().numpy()
    mean_only = select_blocks(w.q, w.k, 128, keep_mean=0.05, keep_radius=0.0)["mask"]
    for kvh in range(2):
        want = {kb for (kv, kb) in planted if kv == kvh}
        assert set(np.nonzero(ref["rad2"][0, kvh] > ref["tau_radius"][0, kvh])[0].tolist()) == want
        for h in range(4 * kvh, 4 * kvh + 4):
            rescued = {kb for kb in range(16) if mask[0, h, :, kb].any() and not mean_only[0, h, :, kb].any()}
            assert rescued <= want


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Tq, Tk, bs, offsets, window, keeps
    (1, 8, 2, 1000, 1000, 64, None, 0, (0.1, 0.1)),
    (2, 8, 2, 300, 900, 128, [600, 100], 0, (0.2, 0.05)),
    (2, 4, 2, 300, 900, 32, [600, 100], 250, (0.3, 0.2)),
    (1, 4, 4, 512, 512, 128, None, 0, (1.0, 0.0)),
    (1, 4, 1, 700, 700, 100, None, 130, (0.0, 0.5)),
])
def test_select_bf16_matches_oracle(case):
    B, Hq, Hkv, Tq, Tk, bs, offs, W, keeps = case
    w = synth.attention_inputs(B, Hq, Hkv, Tq, Tk, 128, torch.bfloat16, seed=Tq + Tk)
    check_select(w.q, w.k, bs, cache_off=offs, window=W, keep_mean=keeps[0], keep_radius=keeps[1])


@pytest.mark.parametrize("d", [16, 64])
def test_select_f32_matches_oracle(d):
    w = synth.attention_inputs(1, 8, 2, 96, 96, d, torch.float32, seed=d)
    check_select(w.q, w.k, 8, keep_mean=0.1, keep_radius=0.1)


def test_select_absolute_threshold_mode():
    w = synth.attention_inputs(1, 8, 2, 640, 640, 128, torch.bfloat16, seed=31)
    ref = select_blocks(w.q, w.k, 64, keep_mean=0.15, keep_radius=0.1)
    got = attn_block_select(dev(w.q), dev(w.k), block_size=64, keep_mean=-1.0, keep_radius=-1.0,
                            tau_mean=torch.tensor(ref["tau_mean"], device="cuda"),
                            tau_radius=torch.tensor(ref["tau_radius"], device="cuda"))
    assert np.array_equal(got["mask"].cpu().numpy(), ref["mask"])


def test_list_from_mask_matches_oracle():
    g = torch.Generator().manual_seed(3)
    mask = (torch.rand((3, 5, 7, 300), generator=g) < 0.3).to(torch.uint8)
    assert lists_match(attn_block_list_from_mask(mask.cuda()), mask.numpy())


def test_block_sparse_prefill_on_selected_blocks():
    w = synth.block_sparse_prefill(T=2048, BS=128, Hq=8, Hkv=2, d=128, frac=0.125)
    sel = attn_block_select(dev(w.q), dev(w.k), block_size=128, keep_mean=0.1, keep_radius=0.125)
    ref_sel = select_blocks(w.q, w.k, 128, keep_mean=0.1, keep_radius=0.125)
    assert np.array_equal(sel["mask"].cpu().numpy(), ref_sel["mask"])
    o = attn_prefill(dev(w.q), dev(w.k), dev(w.v), block_list=sel["list"], block_size=128)
    ref = attend(w.q, w.k, w.v, block_mask=ref_sel["mask"], block_size=128)
    assert max_abs(o, ref) <= BF16_TOL


# ---------------------------------------------------------------- fused selection + prefill
@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Tq, Tk, offsets, window, sink, keeps
    (1, 8, 2, 2048, 2048, None, 0, False, (0.1, 0.125)),       # planted-outlier prompt, one shot
    (3, 8, 2, 300, 1500, [1200, 37, 640], 0, True, (0.1, 0.1)),  # query-chunked: chunks at cache offsets
    (4, 8, 2, 256, 1200, [900, 37, 640, 400], 0, True, (0.1, 0.1)),  # the same, KV groups longest first
    (2, 16, 4, 384, 1400, [1000, 500], 700, True, (0.2, 0.05)),  # chunks with a window
])
def test_fused_block_sparse_prefill(case):
    """attn_block_sparse_prefill, which decides each key block inside the prefill from the
    selection's scores and thresholds, equals the two-call route (attn_block_select, then
    attn_prefill over its mask) bit for bit, writes the same mask when asked, and matches the
    oracle: its selection at the same offsets, then attention over that mask."""
    B, Hq, Hkv, Tq, Tk, offs, W, with_sink, (km, kr) = case
    announce(f"fused block-sparse prefill {case}")
    if offs is None:
        w = synth.block_sparse_prefill(T=Tq, BS=128, Hq=Hq, Hkv=Hkv, d=128, frac=0.125)
        w.cache_off = None
    else:
        w = synth.attention_inputs(B, Hq, Hkv, Tq, Tk, 128, torch.bfloat16, seed=Tq + Tk, with_sink=with_sink,
                                   window=W, cache_off=offs)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    off = None if w.cache_off is None else dev(w.cache_off)
    sink = dev(w.sink) if with_sink else None
    o, sel = attn_block_sparse_prefill(q, k, v, cache_off=off, window=W, sink=sink, keep_mean=km, keep_radius=kr,
                                       want_mask=True)
    o_plain = attn_block_sparse_prefill(q, k, v, cache_off=off, window=W, sink=sink, keep_mean=km, keep_radius=kr)
    two = attn_block_select(q, k, block_size=128, cache_off=off, window=W, keep_mean=km, keep_radius=kr)
    assert torch.equal(sel["mask"], two["mask"])
    o_two = attn_prefill(q, k, v, cache_off=off, window=W, sink=sink, block_mask=two["mask"], block_size=128)
    assert torch.equal(o, o_two) and torch.equal(o_plain, o_two)
    ref_sel = select_blocks(w.q, w.k, 128, cache_off=None if offs is None else offs, window=W, keep_mean=km,
                            keep_radius=kr)
    assert min_gap(ref_sel) > REL_EPS
    assert np.array_equal(sel["mask"].cpu().numpy(), ref_sel["mask"])
    ref = attend(w.q, w.k, w.v, cache_off=w.cache_off, window=W, sink=w.sink if with_sink else None,
                 block_mask=ref_sel["mask"], block_size=128)
    assert max_abs(o, ref) <= BF16_TOL


def test_fused_block_sparse_prefill_f32():
    w = synth.attention_inputs(2, 4, 2, 70, 150, 32, torch.float32, seed=41, with_sink=True, cache_off=[80, 33])
    o, sel = attn_block_sparse_prefill(dev(w.q), dev(w.k), dev(w.v), cache_off=dev(w.cache_off), sink=dev(w.sink),
                                       block_size=16, keep_mean=0.2, keep_radius=0.1, want_mask=True)
    ref_sel = select_blocks(w.q, w.k, 16, cache_off=[80, 33], keep_mean=0.2, keep_radius=0.1)
    assert np.array_equal(sel["mask"].cpu().numpy(), ref_sel["mask"])
    ref = attend(w.q, w.k, w.v, cache_off=w.cache_off, sink=w.sink, block_mask=ref_sel["mask"], block_size=16)
    assert max_abs(o, ref) <= 1e-5
