"""Pins for the float64 attention oracle (CPU only).

Each test ties the oracle to something other than itself: an independent scalar
brute force, a library routine (torch SDPA in float64), a mask figure the pages
print, closed forms, and the equivalences the pages report
(sotaaz.com/post/attention-in-code: decode with a cache equals one shot, GQA
equals MHA with copied KV heads, the ring cache equals the window mask, the
sink's limits; factory.pai-world.com "Attention Variants": the window figure,
window >= n equals full causal, and the ~8x entry count).
"""
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import allowed_pair_count, attend, key_allowed
from oracle.brute import attend_brute
from oracle.ring import RingCache, attend_unmasked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_mask(name):
    window, rows = None, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("window"):
                window = int(line.split()[1])
            else:
                rows.append([int(c) for c in line])
    return window, np.array(rows, dtype=bool)


def _inputs(B, Hq, Hkv, Tq, Tcap, d, seed, sink=False):
    w = synth.attention_inputs(B, Hq, Hkv, Tq, Tcap, d, torch.float32, seed, with_sink=sink)
    return w.q.double(), w.k.double(), w.v.double(), (w.sink.double() if sink else None)


# ---------------------------------------------------------------- brute force
CASES = [
    # B, Hq, Hkv, Tq, Tcap, offsets
    (1, 2, 2, 5, 5, None),        # MHA, square causal
    (1, 4, 2, 3, 9, None),        # GQA, decode-like block at offset 6
    (1, 3, 1, 1, 7, None),        # MQA, single-token decode
    (2, 4, 2, 4, 11, [2, 7]),     # per-sequence offsets (Tk_b = 6 and 11)
    (1, 4, 1, 7, 12, [5]),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("window", [0, 1, 3])
@pytest.mark.parametrize("use_sink", [False, True])
def test_oracle_matches_brute_force(case, window, use_sink):
    B, Hq, Hkv, Tq, Tcap, offs = case
    q, k, v, sink = _inputs(B, Hq, Hkv, Tq, Tcap, 6, seed=11, sink=use_sink)
    o = attend(q, k, v, cache_off=offs, window=window, sink=sink)
    ob = np.array(attend_brute(q, k, v, cache_off=offs, window=window, sink=sink))
    assert np.max(np.abs(o - ob)) <= 1e-13


@pytest.mark.parametrize("bs", [2, 3])
def test_oracle_block_mask_matches_brute_force(bs):
    B, Hq, Hkv, Tq, Tcap = 2, 4, 2, 7, 10
    q, k, v, sink = _inputs(B, Hq, Hkv, Tq, Tcap, 5, seed=3, sink=True)
    rng = np.random.default_rng(5)
    bm = rng.integers(0, 2, size=(B, Hq, -(-Tq // bs), -(-Tcap // bs))).astype(np.uint8)
    for s in (None, sink):
        o = attend(q, k, v, cache_off=[3, 0], window=4, sink=s, block_mask=bm, block_size=bs)
        ob = np.array(attend_brute(q, k, v, cache_off=[3, 0], window=4, sink=s, block_mask=bm,
                                   block_size=bs))
        assert np.max(np.abs(o - ob)) <= 1e-13


def test_empty_rows_are_zero():
    q, k, v, _ = _inputs(1, 2, 1, 4, 4, 3, seed=1)
    bm = np.zeros((1, 2, 2, 2), dtype=np.uint8)
    assert np.all(attend(q, k, v, block_mask=bm, block_size=2) == 0.0)


# ---------------------------------------------------------------- library routine
def test_offset_zero_matches_torch_sdpa_causal():
    q, k, v, _ = _inputs(2, 4, 4, 9, 9, 8, seed=2)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    o = attend(q, k, v, cache_off=[0, 0])
    assert np.max(np.abs(o - ref.numpy())) <= 1e-13


def test_gqa_matches_torch_sdpa_with_explicit_bottom_right_mask():
    # The explicit-mask workaround (tilnote.io note on Express: an explicit attn_mask is
    # needed when the offset is not 0) gives the same result as the offset rule.
    Tq, Tk = 5, 12
    q, k, v, _ = _inputs(1, 6, 2, Tq, Tk, 8, seed=4)
    kk, vv = k.repeat_interleave(3, dim=1), v.repeat_interleave(3, dim=1)
    i = torch.arange(Tk - Tq, Tk)[:, None]
    j = torch.arange(Tk)[None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, attn_mask=(j <= i))
    assert np.max(np.abs(attend(q, k, v) - ref.numpy())) <= 1e-13


def test_top_left_alignment_differs_when_block_is_offset():
    # Block-internal causal masking (the ONNX is_causal behaviour the Express note
    # describes) is only right for a block at position 0.
    Tq, Tk = 4, 10
    q, k, v, _ = _inputs(1, 2, 2, Tq, Tk, 8, seed=5)
    top_left = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).numpy()
    o = attend(q, k, v)
    assert np.max(np.abs(o - top_left)) > 1e-2
    qs, ks, vs, _ = _inputs(1, 2, 2, Tk, Tk, 8, seed=5)
    assert np.max(np.abs(attend(qs, ks, vs) - torch.nn.functional.scaled_dot_product_attention(
        qs, ks, vs, is_causal=True).numpy())) <= 1e-13


# ---------------------------------------------------------------- page invariants
@pytest.mark.parametrize("n_kv", [8, 2, 1])  # MHA, GQA, MQA
def test_decode_token_by_token_equals_one_shot(n_kv):
    w = synth.attention_inputs(1, 8, n_kv, 40, 40, 16, torch.float32, seed=0, with_sink=True)
    q, k, v = w.q.double(), w.k.double(), w.v.double()
    for sink in (None, w.sink.double()):
        full = attend(q, k, v, sink=sink)
        worst = 0.0
        for t in range(40):
            step = attend(q[:, :, t:t + 1], k[:, :, :t + 1], v[:, :, :t + 1], cache_off=[t], sink=sink)
            worst = max(worst, float(np.max(np.abs(step[:, :, 0] - full[:, :, t]))))
        assert worst <= 1e-13
        # a chunked prefill at uneven offsets gives the same rows
        for a, b in ((0, 7), (7, 20), (20, 40)):
            part = attend(q[:, :, a:b], k[:, :, :b], v[:, :, :b], cache_off=[a], sink=sink)
            assert np.max(np.abs(part - full[:, :, a:b])) <= 1e-13
        # and the same chunk read from a larger cache (rows beyond Tk_b are never used)
        pad = torch.full((1, n_kv, 5, 16), float("nan"), dtype=torch.float64)
        part = attend(q[:, :, 7:20], torch.cat([k[:, :, :20], pad], 2), torch.cat([v[:, :, :20], pad], 2),
                      cache_off=[7], sink=sink)
        assert np.max(np.abs(part - full[:, :, 7:20])) <= 1e-13


def test_gqa_equals_mha_with_kv_copied_per_group():
    w = synth.tiny(seed=1)
    q, k2, v2 = w.q.double(), w.k.double(), w.v.double()      # 8 query heads, 2 KV heads
    k8, v8 = k2.repeat_interleave(4, dim=1), v2.repeat_interleave(4, dim=1)
    assert np.max(np.abs(attend(q, k2, v2) - attend(q, k8, v8))) <= 1e-13
    # head h reads KV head h // g, not h % n_kv
    k8w, v8w = k2.repeat(1, 4, 1, 1), v2.repeat(1, 4, 1, 1)
    assert np.max(np.abs(attend(q, k2, v2) - attend(q, k8w, v8w))) > 1e-3


def test_ring_cache_equals_window_mask_every_step():
    W, T = 8, 50
    w = synth.attention_inputs(1, 8, 2, T, T, 16, torch.float32, seed=7, with_sink=True)
    q, k, v, sink = w.q.double()[0].numpy(), w.k.double()[0].numpy(), w.v.double()[0].numpy(), w.sink.double().numpy()
    full = attend(q[None], k[None], v[None], window=W, sink=sink)[0]
    ring = RingCache(2, 16, W)
    worst = 0.0
    for t in range(T):
        K, V = ring.add(k[:, t], v[:, t])
        o = attend_unmasked(q[:, t], K, V, 8, sink=sink)
        worst = max(worst, float(np.max(np.abs(o - full[:, t]))))
    assert worst <= 1e-13
    # token 0's value changed by 100: every step from W on is exactly unchanged
    v2 = v.copy()
    v2[:, 0] += 100.0
    full2 = attend(q[None], k[None], v2[None], window=W, sink=sink)[0]
    assert np.array_equal(full2[:, W:], full[:, W:])
    assert np.max(np.abs(full2[:, :W] - full[:, :W])) > 1.0


def test_window_at_least_n_is_bitwise_causal():
    q, k, v, sink = _inputs(1, 4, 2, 12, 12, 8, seed=8, sink=True)
    causal = attend(q, k, v, sink=sink)
    for W in (12, 13, 100):
        assert np.array_equal(attend(q, k, v, window=W, sink=sink), causal)


@pytest.mark.parametrize("fname", ["causal_mask_n8.txt", "swa_mask_n8_w4.txt"])
def test_mask_rule_reproduces_page_figure(fname):
    window, fig = _load_mask(fname)
    i = np.arange(8)[:, None]
    j = np.arange(8)[None, :]
    assert np.array_equal(key_allowed(i, j, window), fig)


def test_window_one_sees_only_itself():
    q, k, v, _ = _inputs(1, 2, 2, 6, 6, 4, seed=9)
    assert np.max(np.abs(attend(q, k, v, window=1) - v.numpy())) <= 1e-15


def test_window_entry_count_matches_page():
    with open(os.path.join(GOLDEN, "swa_counts.txt")) as f:
        n, W, approx, exact = [int(x) for x in [l for l in f if not l.startswith("#")][0].split()]
    count = allowed_pair_count(n, n, W)
    assert count == exact == W * (W + 1) // 2 + (n - W) * W
    assert 0.75 * approx <= n * n / count <= 1.25 * approx  # "about 8x fewer" than full


def test_sink_closed_form_and_limits():
    w = synth.tiny(seed=3, with_sink=True)
    q, k, v, sink = w.q.double(), w.k.double(), w.v.double(), w.sink.double()
    plain, lse = attend(q, k, v, return_lse=True)
    with_sink = attend(q, k, v, sink=sink)
    factor = 1.0 / (1.0 + np.exp(sink.numpy()[None, :, None] - lse))
    assert np.max(np.abs(with_sink - plain * factor[..., None])) <= 1e-13
    # sink = -inf is exactly plain attention
    assert np.array_equal(attend(q, k, v, sink=torch.full((8,), -math.inf, dtype=torch.float64)), plain)
    # with v = 1 the output is the total weight on real keys: strictly below 1 with a sink
    ones = torch.ones_like(v)
    total = attend(q, k, ones, sink=sink)[..., 0]
    assert np.all(total < 1.0) and np.max(np.abs(total - factor)) <= 1e-13
    assert np.max(np.abs(attend(q, k, ones)[..., 0] - 1.0)) <= 1e-14
    # a sink far above every score sends almost all weight to the empty slot
    big = attend(q, k, v, sink=torch.full((8,), 20.0, dtype=torch.float64))
    ratio = np.abs(big).max() / np.abs(plain).max()
    assert ratio < 1e-5


def test_block_mask_all_kept_equals_dense_bitwise():
    q, k, v, sink = _inputs(2, 4, 2, 9, 13, 8, seed=10, sink=True)
    bm = np.ones((2, 4, 3, 4), dtype=np.uint8)
    for s in (None, sink):
        dense = attend(q, k, v, cache_off=[4, 2], window=5, sink=s)
        sparse = attend(q, k, v, cache_off=[4, 2], window=5, sink=s, block_mask=bm, block_size=4)
        assert np.array_equal(dense, sparse)


def test_row_subsets_match_full():
    q, k, v, sink = _inputs(1, 4, 2, 20, 20, 8, seed=12, sink=True)
    full = attend(q, k, v, window=6, sink=sink, row_block=7)
    sub = attend(q, k, v, window=6, sink=sink, rows=[0, 5, 19], heads=[1, 3])
    assert np.array_equal(sub, full[:, [1, 3]][:, :, [0, 5, 19]])
