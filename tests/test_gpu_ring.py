"""GPU parity of attn_ring_decode (sliding-window decode over a W-slot ring cache with the
step's K/V appended by the call) against the float64 oracle, through the C ABI.

Two independent oracle routes: the oracle's own ring (slot n mod W, unmasked attention
over the filled slots) and masked attention with window W over the whole history.  The
ring's contents after each step are compared bit for bit (the append is a copy)."""
import numpy as np
import pytest
import torch

import synth
from oracle import attend
from oracle.ring import RingCache, attend_unmasked
from sparse_offset_causal_amd import AttnError, attn_ring_decode
from tests.gpu_helpers import BF16_TOL, F32_TOL, announce, dev, host64, max_abs, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("with_sink", [False, True])
@pytest.mark.parametrize("split", [0, 3])
def test_ring_decode_f32_steps_match_both_oracle_routes(with_sink, split):
    announce(f"ring f32 sink={with_sink} split={split}")
    B, Hq, Hkv, d, W, steps = 2, 8, 2, 16, 8, 40
    st = synth.ring_state(B, Hq, Hkv, d, W, n_lo=0, n_hi=0, seed=3, dtype=torch.float32)
    sink = st.sink if with_sink else None
    k_ring, v_ring, n_seen = dev(st.k), dev(st.v), dev(st.n_seen)
    rings = [RingCache(Hkv, d, W) for _ in range(B)]
    hist_q, hist_k, hist_v = [], [], []
    worst_ring = worst_mask = 0.0
    for t in range(steps):
        q, kn, vn = synth.ring_step(B, Hq, Hkv, d, t, seed=3, dtype=torch.float32)
        o = attn_ring_decode(dev(q), dev(kn), dev(vn), k_ring, v_ring, n_seen, sink=dev(sink), split_tokens=split)
        n_seen += 1
        hist_q.append(q)
        hist_k.append(kn)
        hist_v.append(vn)
        for b in range(B):
            K, V = rings[b].add(host64(kn[b, :, 0]), host64(vn[b, :, 0]))
            ref = attend_unmasked(host64(q[b, :, 0]), K, V, Hq, sink=None if sink is None else host64(sink))
            worst_ring = max(worst_ring, max_abs(o[b, :, 0], ref))
            filled = min(t + 1, W)
            assert np.array_equal(host64(k_ring[b, :, :filled]), rings[b].k[:, :filled])
            assert np.array_equal(host64(v_ring[b, :, :filled]), rings[b].v[:, :filled])
        # masked route: the step's row at position t of the whole history, window W
        kh, vh = torch.cat(hist_k, 2), torch.cat(hist_v, 2)
        ref_m = attend(q, kh, vh, cache_off=[t] * B, window=W, sink=sink)
        worst_mask = max(worst_mask, max_abs(o, ref_m))
    assert worst_ring <= F32_TOL and worst_mask <= F32_TOL, (worst_ring, worst_mask)


@pytest.mark.parametrize("split,with_sink", [(24, True), (32, True), (64, True), (32, False)])
def test_ring_decode_bf16_staggered_sequences(split, with_sink):
    """split 24: three splits per ring (split kernel + merge kernel); 32: two splits merged
    inside one workgroup; 64: one split, its workgroup's second wave empty."""
    announce(f"ring bf16 staggered split={split} sink={with_sink}")
    B, Hq, Hkv, d, W = 3, 32, 8, 128, 64
    # empty, partly filled and wrapped rings; unwritten slots hold stale values
    st = synth.ring_state(B, Hq, Hkv, d, W, seed=5, n_seen=[0, 37, 300])
    k_ring, v_ring, n_seen = dev(st.k), dev(st.v), dev(st.n_seen)
    sink = dev(st.sink) if with_sink else None
    sink64 = host64(st.sink) if with_sink else None
    rings = []
    for b in range(B):
        r = RingCache(Hkv, d, W)
        r.k, r.v, r.n = host64(st.k[b]), host64(st.v[b]), int(st.n_seen[b])
        rings.append(r)
    worst = 0.0
    for t in range(90):
        q, kn, vn = synth.ring_step(B, Hq, Hkv, d, t, seed=5)
        o = attn_ring_decode(dev(q), dev(kn), dev(vn), k_ring, v_ring, n_seen, sink=sink, split_tokens=split)
        n_seen += 1
        for b in range(B):
            K, V = rings[b].add(host64(kn[b, :, 0]), host64(vn[b, :, 0]))
            worst = max(worst, max_abs(o[b, :, 0], attend_unmasked(host64(q[b, :, 0]), K, V, Hq, sink=sink64)))
    for b in range(B):
        filled = min(rings[b].n, W)
        assert np.array_equal(host64(k_ring[b, :, :filled]), rings[b].k[:, :filled])
        assert np.array_equal(host64(v_ring[b, :, :filled]), rings[b].v[:, :filled])
    assert worst <= BF16_TOL, worst
    assert torch.equal(n_seen.cpu(), st.n_seen + 90)


@pytest.mark.parametrize("split", [0, 300])
def test_ring_decode_full_size_B64_W1024(split):
    announce(f"ring full size split={split}")
    B, Hq, Hkv, d, W = 64, 32, 8, 128, 1024
    st = synth.ring_state(B, Hq, Hkv, d, W, n_lo=0, n_hi=4096, seed=7)
    q, kn, vn = synth.ring_step(B, Hq, Hkv, d, 0, seed=7)
    k_ring, v_ring = dev(st.k), dev(st.v)
    o = attn_ring_decode(dev(q), dev(kn), dev(vn), k_ring, v_ring, dev(st.n_seen), sink=dev(st.sink),
                         split_tokens=split)
    kr, vr = host64(k_ring), host64(v_ring)
    worst = 0.0
    for b in range(B):
        r = RingCache(Hkv, d, W)
        r.k, r.v, r.n = host64(st.k[b]), host64(st.v[b]), int(st.n_seen[b])
        K, V = r.add(host64(kn[b, :, 0]), host64(vn[b, :, 0]))
        assert np.array_equal(kr[b], r.k) and np.array_equal(vr[b], r.v)
        worst = max(worst, max_abs(o[b, :, 0], attend_unmasked(host64(q[b, :, 0]), K, V, Hq, sink=host64(st.sink))))
    assert worst <= BF16_TOL, worst


def test_ring_decode_rejects_multi_row_queries():
    st = synth.ring_state(1, 8, 2, 128, 64, n_lo=0, n_hi=0, seed=1)
    q = torch.zeros(1, 8, 2, 128, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(1, 2, 1, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AttnError, match="tq = 1"):
        attn_ring_decode(q, kn, kn, dev(st.k), dev(st.v), dev(st.n_seen))
