"""GPU parity of attn_prefill / attn_decode against the float64 oracle (through the C ABI).

Sizes span several 128-row query tiles and 64/128-key KV tiles with ragged tails,
per-sequence cache offsets, windows, sinks and GQA/MQA/MHA groupings.  Bar: max-abs
2e-2 for bf16 inputs, 1e-5 for the float32 path; invariants are checked bitwise.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import attend
from sparse_offset_causal_amd import AttnError, attn_block_list_from_mask, attn_decode, attn_prefill
from tests.gpu_helpers import BF16_TOL, F32_TOL, announce, dev, host64, max_abs, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_prefill(w, **kw):
    return attn_prefill(dev(w.q), dev(w.k), dev(w.v), cache_off=dev(w.cache_off), window=w.window,
                        sink=dev(w.sink), scale=w.scale, **kw)


def oracle_of(w, **kw):
    return attend(w.q, w.k, w.v, cache_off=w.cache_off, window=w.window, sink=w.sink, scale=w.scale, **kw)


# ---------------------------------------------------------------- tiny float32 case
@pytest.mark.parametrize("with_sink", [False, True])
@pytest.mark.parametrize("window", [0, 8])
def test_tiny_f32_prefill_and_token_by_token_decode(with_sink, window):
    announce(f"tiny f32 sink={with_sink} window={window}")
    w = synth.tiny(seed=0, with_sink=with_sink, window=window)
    ref = oracle_of(w)
    o = run_prefill(w)
    assert max_abs(o, ref) <= F32_TOL
    qd, kd, vd, sd = dev(w.q), dev(w.k), dev(w.v), dev(w.sink)
    for split in (0, 8, 13):
        worst = 0.0
        for t in range(40):
            off = torch.tensor([t], dtype=torch.int32, device="cuda")
            step = attn_decode(qd[:, :, t:t + 1], kd, vd, cache_off=off, window=window, sink=sd, split_tokens=split)
            worst = max(worst, max_abs(step[:, :, 0], ref[:, :, t]))
            step_p = attn_prefill(qd[:, :, t:t + 1], kd, vd, cache_off=off, window=window, sink=sd)
            worst = max(worst, max_abs(step_p[:, :, 0], ref[:, :, t]))
        assert worst <= F32_TOL, (split, worst)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_f32_other_head_dims(d):
    w = synth.attention_inputs(2, 4, 2, 33, 70, d, torch.float32, seed=d, with_sink=True, window=20,
                               cache_off=[37, 10])
    assert max_abs(run_prefill(w), oracle_of(w)) <= F32_TOL
    ref = attend(w.q[:, :, :3], w.k, w.v, cache_off=[37, 10], window=20, sink=w.sink)
    o = attn_decode(dev(w.q[:, :, :3]), dev(w.k), dev(w.v), cache_off=dev(w.cache_off), window=20,
                    sink=dev(w.sink), split_tokens=16)
    assert max_abs(o, ref) <= F32_TOL


# ---------------------------------------------------------------- bf16 prefill
PREFILL_CASES = [
    # B, Hq, Hkv, Tq, Tk, offsets, window, sink
    (1, 8, 2, 300, 300, None, 0, False),
    (2, 8, 2, 200, 700, None, 0, True),
    (2, 4, 4, 129, 1000, [300, 871], 0, True),
    (1, 8, 1, 640, 640, None, 200, True),
    (1, 6, 2, 1, 777, None, 0, True),
    (1, 8, 2, 64, 64, None, 1, False),
    (3, 8, 8, 190, 450, [0, 100, 260], 77, True),
    (1, 16, 8, 1024, 1536, None, 0, False),
    # windowed GQA: g = 2 and g = 6 stack two heads over 64 rows, g = 3 stacks rows only
    (2, 4, 2, 333, 900, [100, 567], 150, True),
    (1, 12, 2, 200, 500, [300], 64, True),
    (1, 6, 2, 250, 250, None, 40, False),
    # chunks at different cache lengths on the KV-group-per-XCD grid: the groups run longest
    # sequence first (equal offsets, and a full 64-sequence batch)
    (8, 4, 1, 130, 700, [570, 3, 300, 129, 64, 570, 0, 411], 0, True),
    (64, 2, 1, 16, 200, [(37 * i) % 185 for i in range(64)], 0, False),
    # 65 sequences: past the ranked order's one-wave limit the groups keep sequence order
    (65, 8, 8, 3, 90, [(29 * i) % 88 for i in range(65)], 0, True),
]


@pytest.mark.parametrize("case", PREFILL_CASES)
def test_bf16_prefill_matches_oracle(case):
    B, Hq, Hkv, Tq, Tk, offs, W, with_sink = case
    announce(f"bf16 prefill {case}")
    w = synth.attention_inputs(B, Hq, Hkv, Tq, Tk, 128, torch.bfloat16, seed=sum(case[:5]), with_sink=with_sink,
                               window=W, cache_off=offs)
    o = run_prefill(w)
    err = max_abs(o, oracle_of(w))
    assert err <= BF16_TOL, err


# Windowed GQA on the grid that gives each XCD whole KV groups (batch x n_kv a multiple of 8):
# the launch the window workload is timed in.  g = 4 stacks four heads over 32 rows, g = 2 two
# heads over 64 rows; every element is compared.
STACKED_CASES = [
    # B, Hq, Hkv, Tq, Tk, offsets, window
    (2, 16, 4, 700, 1300, [600, 37], 150),
    (4, 8, 4, 333, 900, [0, 567, 200, 301], 150),
    (1, 32, 8, 257, 2000, [1743], 1024),
    (2, 16, 4, 64, 700, [636, 5], 7),
]


@pytest.mark.parametrize("case", STACKED_CASES)
def test_bf16_window_gqa_stacked_heads_xcd_grouped(case):
    B, Hq, Hkv, Tq, Tk, offs, W = case
    announce(f"bf16 windowed GQA, stacked heads on the XCD-grouped grid {case}")
    assert (B * Hkv) % 8 == 0 and (Hq // Hkv) % 2 == 0
    w = synth.attention_inputs(B, Hq, Hkv, Tq, Tk, 128, torch.bfloat16, seed=Tq + W, with_sink=True, window=W,
                               cache_off=offs)
    o = run_prefill(w)
    err = max_abs(o, oracle_of(w))
    assert err <= BF16_TOL, err


def test_bf16_prefill_strided_views():
    # q/k/v/o as views into larger buffers (head-major and token-major layouts)
    base = synth.normal((1, 300, 12, 128), 5, torch.bfloat16)  # [B, T, H, d] layout
    q = base[:, :, :8].permute(0, 2, 1, 3)
    k = base[:, :, 8:10].permute(0, 2, 1, 3)
    v = base[:, :, 10:12].permute(0, 2, 1, 3)
    ref = attend(q, k, v, window=50)
    out = torch.zeros((1, 300, 8, 128), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    attn_prefill(dev(base)[:, :, :8].permute(0, 2, 1, 3), dev(base)[:, :, 8:10].permute(0, 2, 1, 3),
                 dev(base)[:, :, 10:12].permute(0, 2, 1, 3), window=50, out=out)
    assert max_abs(out, ref) <= BF16_TOL


def test_bf16_window_at_least_tk_is_bitwise_causal_and_sink_neg_inf_is_plain():
    w = synth.attention_inputs(1, 8, 2, 333, 500, 128, torch.bfloat16, seed=3)
    causal = run_prefill(w)
    for W in (500, 501, 10 ** 6):
        w.window = W
        assert torch.equal(run_prefill(w), causal)
    w.window = 0
    w.sink = torch.full((8,), -math.inf)
    assert torch.equal(run_prefill(w), causal)


def test_bf16_masked_keys_never_matter_bitwise():
    # Keys a row may not see (future keys of the block, keys before the window, and cache rows
    # beyond Tk_b) are overwritten with large finite values: the output must not change at all.
    B, Hq, Hkv, Tq, cap, W = 2, 8, 2, 200, 900, 150
    offs = [400, 650]
    w = synth.attention_inputs(B, Hq, Hkv, Tq, cap, 128, torch.bfloat16, seed=4, with_sink=True, window=W,
                               cache_off=offs)
    o1 = run_prefill(w)
    k2, v2 = w.k.clone(), w.v.clone()
    for b, off in enumerate(offs):
        tkb = off + Tq
        k2[b, :, tkb:] = 3e4
        v2[b, :, tkb:] = -3e4
        first_visible = off - W + 1  # smallest key any row of the block sees
        k2[b, :, :first_visible] = 3e4
        v2[b, :, :first_visible] = 3e4
    w.k, w.v = k2, v2
    o2 = run_prefill(w)
    assert torch.equal(o1, o2)


def test_bf16_deterministic_and_top_left_alignment_differs():
    w = synth.attention_inputs(1, 8, 2, 256, 1024, 128, torch.bfloat16, seed=6)
    o1, o2 = run_prefill(w), run_prefill(w)
    assert torch.equal(o1, o2)
    # block-internal causal masking (as if the block started at position 0) differs
    top_left = attend(w.q, w.k[:, :, :256], w.v[:, :, :256])
    assert max_abs(o1, top_left) > 0.1


def test_bf16_block_list_all_kept_equals_dense_bitwise():
    B, Hq, Hkv, Tq, Tk = 2, 8, 2, 384, 1000
    w = synth.attention_inputs(B, Hq, Hkv, Tq, Tk, 128, torch.bfloat16, seed=7, with_sink=True, window=300,
                               cache_off=[616, 200])
    dense = run_prefill(w)
    mask = torch.ones((B, Hq, 3, 8), dtype=torch.uint8, device="cuda")
    lst = attn_block_list_from_mask(mask)
    sparse = run_prefill(w, block_list=lst, block_size=128)
    assert torch.equal(dense, sparse)


def test_bf16_block_list_random_mask_matches_oracle():
    B, Hq, Hkv, Tq, Tk = 2, 8, 2, 500, 900
    w = synth.attention_inputs(B, Hq, Hkv, Tq, Tk, 128, torch.bfloat16, seed=8, with_sink=False, window=0,
                               cache_off=[400, 100])
    g = torch.Generator().manual_seed(9)
    mask = (torch.rand((B, Hq, 4, 8), generator=g) < 0.4).to(torch.uint8)
    mask[0, 0, 1] = 0  # an empty query block: its rows are 0
    lst = attn_block_list_from_mask(mask.cuda())
    o = run_prefill(w, block_list=lst, block_size=128)
    ref = oracle_of(w, block_mask=mask.numpy(), block_size=128)
    assert max_abs(o, ref) <= BF16_TOL
    assert torch.count_nonzero(o[0, 0, 128:256]) == 0


@pytest.mark.parametrize("window,with_sink", [(0, False), (150, True), (333, False)])
def test_bf16_block_mask_matches_block_list_and_oracle(window, with_sink):
    """The block mask walked in the kernel selects the same tiles as its kept-block list (so the
    two outputs are bitwise equal) and matches the oracle.  The mask marks future and
    out-of-window blocks too (the causal and window rules still apply inside kept blocks) and
    leaves one query block empty; offsets put the window edge and the last row mid-block."""
    announce(f"bf16 block mask window={window} sink={with_sink}")
    B, Hq, Hkv, Tq, Tk = 2, 8, 2, 500, 1300
    offs = [800, 77]
    w = synth.attention_inputs(B, Hq, Hkv, Tq, Tk, 128, torch.bfloat16, seed=31 + window, with_sink=with_sink,
                               window=window, cache_off=offs)
    g = torch.Generator().manual_seed(32 + window)
    mask = (torch.rand((B, Hq, 4, 11), generator=g) < 0.45).to(torch.uint8)
    mask[1, 3, 2] = 0
    mask[0, 5] = 1
    md = mask.cuda()
    o_mask = run_prefill(w, block_mask=md, block_size=128)
    o_list = run_prefill(w, block_list=attn_block_list_from_mask(md), block_size=128)
    assert torch.equal(o_mask, o_list)
    ref = oracle_of(w, block_mask=mask.numpy(), block_size=128)
    assert max_abs(o_mask, ref) <= BF16_TOL
    if not with_sink:
        assert torch.count_nonzero(o_mask[1, 3, 256:384]) == 0
    ones = torch.ones_like(md)
    assert torch.equal(run_prefill(w, block_mask=ones, block_size=128), run_prefill(w))


def test_f32_block_mask_matches_oracle():
    w = synth.attention_inputs(2, 4, 2, 70, 130, 32, torch.float32, seed=33, with_sink=True, window=50,
                               cache_off=[60, 10])
    g = torch.Generator().manual_seed(34)
    mask = (torch.rand((2, 4, 5, 9), generator=g) < 0.5).to(torch.uint8)
    o = run_prefill(w, block_mask=mask.cuda(), block_size=16)
    assert max_abs(o, oracle_of(w, block_mask=mask.numpy(), block_size=16)) <= F32_TOL


# ---------------------------------------------------------------- bf16 decode
@pytest.mark.parametrize("tq", [1, 2, 8])
@pytest.mark.parametrize("split", [0, 256, 1000])
def test_bf16_decode_matches_oracle_and_prefill(tq, split):
    announce(f"bf16 decode tq={tq} split={split}")
    B, Hq, Hkv = 5, 32, 8
    lengths = [1, 130, 1023, 2500, 4000]
    cap = max(lengths) + tq
    w = synth.attention_inputs(B, Hq, Hkv, tq, cap, 128, torch.bfloat16, seed=10 + tq, with_sink=True,
                               cache_off=lengths)
    ref = oracle_of(w)
    o = attn_decode(dev(w.q), dev(w.k), dev(w.v), cache_off=dev(w.cache_off), sink=dev(w.sink), split_tokens=split)
    assert max_abs(o, ref) <= BF16_TOL
    assert max_abs(o, run_prefill(w)) <= BF16_TOL


def test_bf16_decode_window_and_mqa():
    B, Hq, Hkv, tq = 3, 8, 1, 4
    lengths = [50, 700, 2049]
    w = synth.attention_inputs(B, Hq, Hkv, tq, 2100, 128, torch.bfloat16, seed=21, with_sink=True, window=333,
                               cache_off=lengths)
    o = attn_decode(dev(w.q), dev(w.k), dev(w.v), cache_off=dev(w.cache_off), window=333, sink=dev(w.sink),
                    split_tokens=128)
    assert max_abs(o, oracle_of(w)) <= BF16_TOL


@pytest.mark.parametrize("tq,window,split", [(1, 0, 128), (1, 700, 128), (4, 1000, 96), (2, 0, 300)])
def test_bf16_decode_longest_first_order(tq, window, split):
    """Grids of several rounds of the chip take the splits longest first (full, then partial by
    size, then the empty ones below a window); every split must still be computed exactly once.
    70 sequences (two 64-lane chunks of the work-order prefix sums), lengths on split edges."""
    announce(f"bf16 decode longest-first tq={tq} window={window} split={split}")
    B, Hq, Hkv = 70, 8, 2
    g = torch.Generator().manual_seed(40 + tq)
    lengths = torch.randint(1, 3000, (B,), generator=g).tolist()
    lengths[:8] = [1, split - 1, split, split + 1, 2 * split, 2999, 31, 33]
    cap = 3000 + tq
    nsplit = -(-cap // split)
    assert B * Hkv * nsplit > 6 * torch.cuda.get_device_properties(0).multi_processor_count
    w = synth.attention_inputs(B, Hq, Hkv, tq, cap, 128, torch.bfloat16, seed=50 + tq, with_sink=True,
                               window=window, cache_off=lengths)
    o = attn_decode(dev(w.q), dev(w.k), dev(w.v), cache_off=dev(w.cache_off), window=window, sink=dev(w.sink),
                    split_tokens=split)
    assert max_abs(o, oracle_of(w)) <= BF16_TOL


def test_bf16_decode_rejects_too_many_rows():
    w = synth.attention_inputs(1, 32, 4, 8, 64, 128, torch.bfloat16, seed=1)
    with pytest.raises(AttnError, match="32 query rows"):
        attn_decode(dev(w.q), dev(w.k), dev(w.v))
