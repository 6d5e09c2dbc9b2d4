"""Run-twice determinism of every entry point that takes a workspace, with the workspace
filled with 0xff bytes before each call (NaN as float32 and float64, all ones as counters):
the second call must reproduce the first bit for bit, so no result may depend on workspace
contents left by an earlier call.  Each first result is also checked against the float64
oracle, so equal-but-wrong outputs cannot pass."""
import numpy as np
import pytest
import torch

import synth
from oracle import attend, select_blocks
from oracle.mla import mla_absorbed
from oracle.ring import RingCache, attend_unmasked
from sparse_offset_causal_amd import (attn_block_select, attn_block_select_workspace_bytes, attn_decode,
                                      attn_decode_workspace_bytes, attn_dsa_decode, attn_dsa_decode_workspace_bytes,
                                      attn_mla_decode, attn_mla_decode_workspace_bytes, attn_ring_decode,
                                      attn_ring_decode_workspace_bytes)
from tests.gpu_helpers import BF16_TOL, announce, dev, host64, max_abs, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def poisoned(nbytes):
    """A workspace of nbytes with every byte 0xff."""
    return torch.full((max(int(nbytes), 1),), 0xFF, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("split", [0, 96])
def test_decode_twice_with_poisoned_workspace(split):
    announce(f"determinism: decode split={split}")
    w = synth.attention_inputs(5, 32, 8, 2, 3100, 128, torch.bfloat16, seed=61, with_sink=True, window=900,
                               cache_off=[0, 100, 1500, 3000, 2047])
    q, k, v, off, sink = dev(w.q), dev(w.k), dev(w.v), dev(w.cache_off), dev(w.sink)
    need = attn_decode_workspace_bytes(q, k, split)
    outs = []
    for _ in range(2):
        outs.append(attn_decode(q, k, v, cache_off=off, window=900, sink=sink, split_tokens=split,
                                workspace=poisoned(need)))
    assert torch.equal(outs[0], outs[1])
    ref = attend(w.q, w.k, w.v, cache_off=w.cache_off, window=900, sink=w.sink)
    assert max_abs(outs[0], ref) <= BF16_TOL


@pytest.mark.parametrize("split", [0, 24])
def test_ring_decode_twice_with_poisoned_workspace(split):
    announce(f"determinism: ring decode split={split}")
    B, Hq, Hkv, d, W = 3, 32, 8, 128, 64
    st = synth.ring_state(B, Hq, Hkv, d, W, seed=62, n_seen=[0, 37, 300])
    q, kn, vn = synth.ring_step(B, Hq, Hkv, d, 0, seed=62)
    need = attn_ring_decode_workspace_bytes(dev(q), dev(st.k), split)
    res = []
    for _ in range(2):
        kr, vr = dev(st.k), dev(st.v)
        o = attn_ring_decode(dev(q), dev(kn), dev(vn), kr, vr, dev(st.n_seen), sink=dev(st.sink),
                             split_tokens=split, workspace=poisoned(need))
        res.append((o, kr, vr))
    assert all(torch.equal(a, b) for a, b in zip(res[0], res[1]))
    worst = 0.0
    for b in range(B):
        r = RingCache(Hkv, d, W)
        r.k, r.v, r.n = host64(st.k[b]), host64(st.v[b]), int(st.n_seen[b])
        K, V = r.add(host64(kn[b, :, 0]), host64(vn[b, :, 0]))
        worst = max(worst, max_abs(res[0][0][b, :, 0], attend_unmasked(host64(q[b, :, 0]), K, V, Hq,
                                                                        sink=host64(st.sink))))
    assert worst <= BF16_TOL, worst


def test_mla_decode_twice_with_poisoned_workspace():
    announce("determinism: MLA decode")
    c = synth.mla_cache(B=3, H=16, lengths=[5, 1500, 2100], tq=2, seed=63)
    args = [dev(t) for t in (c.q_nope, c.q_rope, c.c_kv, c.k_rope, c.w_uk, c.w_uv)]
    need = attn_mla_decode_workspace_bytes(args[0], args[1], args[2], args[3], args[5], 256)
    outs = [attn_mla_decode(*args, cache_off=dev(c.cache_off), split_tokens=256, workspace=poisoned(need))
            for _ in range(2)]
    assert torch.equal(outs[0], outs[1])
    ref = mla_absorbed(c.q_nope, c.q_rope, c.c_kv, c.k_rope, c.w_uk, c.w_uv, cache_off=c.cache_off)
    assert max_abs(outs[0], ref) <= BF16_TOL


def test_dsa_decode_twice_with_poisoned_workspace():
    announce("determinism: top-k sparse decode")
    x = synth.dsa_inputs(B=3, Hq=32, Hkv=8, tq=2, lengths=[40, 900, 2500], Hi=32, seed=64)
    args = [dev(t) for t in (x.q, x.k, x.v, x.qi, x.ki, x.wi)]
    need = attn_dsa_decode_workspace_bytes(args[0], args[1], 300, 64)
    res = [attn_dsa_decode(*args, 300, cache_off=dev(x.cache_off), sink=dev(x.sink), split_tokens=64,
                           want_kept=True, workspace=poisoned(need)) for _ in range(2)]
    o0, kl0, kc0 = res[0]
    o1, kl1, kc1 = res[1]
    assert torch.equal(o0, o1) and torch.equal(kc0, kc1)
    for b in range(3):
        for t in range(2):
            n = int(kc0[b, t])
            assert torch.equal(kl0[b, t, :n], kl1[b, t, :n])
    # the output over the GPU's own kept lists
    mask = np.zeros((3, 32, 2, x.k.shape[2]), dtype=bool)
    kl, kc = kl0.cpu().numpy(), kc0.cpu().numpy()
    for b in range(3):
        for t in range(2):
            mask[b, :, t, kl[b, t, :kc[b, t]]] = True
    ref = attend(x.q, x.k, x.v, cache_off=x.cache_off, sink=x.sink, block_mask=mask, block_size=1)
    assert max_abs(o0, ref) <= BF16_TOL


def test_block_select_twice_with_poisoned_workspace():
    announce("determinism: block selection")
    w = synth.block_sparse_prefill(T=1536, BS=128, Hq=8, Hkv=2, d=128, frac=0.125)
    q, k = dev(w.q), dev(w.k)
    need = attn_block_select_workspace_bytes(q, k, 128)
    res = [attn_block_select(q, k, block_size=128, keep_mean=0.1, keep_radius=0.125, workspace=poisoned(need))
           for _ in range(2)]
    for key in ("mask", "tau_mean", "tau_radius"):
        assert torch.equal(res[0][key], res[1][key]), key
    lists = [r["list"].cpu().numpy() for r in res]
    assert np.array_equal(lists[0][..., 0], lists[1][..., 0])
    for idx in np.ndindex(*lists[0].shape[:-1]):
        n = lists[0][idx][0]
        assert np.array_equal(lists[0][idx][1:1 + n], lists[1][idx][1:1 + n])
    ref = select_blocks(w.q, w.k, 128, keep_mean=0.1, keep_radius=0.125)
    assert np.array_equal(res[0]["mask"].cpu().numpy(), ref["mask"])
