"""GPU parity of attn_mla_decode (multi-head latent attention, absorbed form) against the
float64 oracle of both forms (oracle/mla.py), through the C ABI.  Inputs are bf16; the
kernel rounds the folded query and the probabilities to bf16 and accumulates in fp32:
bar max-abs 2e-2 on unit-scale outputs."""
import numpy as np
import pytest
import torch

import synth
from oracle.mla import mla_absorbed, mla_naive
from sparse_offset_causal_amd import AttnError, attn_mla_decode
from tests.gpu_helpers import BF16_TOL, announce, dev, max_abs, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run(m, **kw):
    return attn_mla_decode(dev(m.q_nope), dev(m.q_rope), dev(m.c_kv), dev(m.k_rope), dev(m.w_uk), dev(m.w_uv),
                           cache_off=dev(m.cache_off), **kw)


def ref(m, batches=None):
    sl = slice(None) if batches is None else batches
    args = (m.q_nope[sl], m.q_rope[sl], m.c_kv[sl], m.k_rope[sl], m.w_uk, m.w_uv)
    return mla_absorbed(*args, cache_off=m.cache_off[sl])


@pytest.mark.parametrize("split", [0, 64, 1000])
def test_mla_decode_matches_both_oracle_forms(split):
    announce(f"mla decode split={split}")
    m = synth.mla_cache(B=4, H=16, lengths=[0, 1, 100, 1500], seed=1)
    o = run(m, split_tokens=split)
    a = ref(m)
    n = mla_naive(m.q_nope, m.q_rope, m.c_kv, m.k_rope, m.w_uk, m.w_uv, cache_off=m.cache_off)
    assert np.max(np.abs(a - n)) < 1e-12
    assert max_abs(o, a) <= BF16_TOL


@pytest.mark.parametrize("H,tq", [(16, 2), (8, 1), (16, 3), (4, 5)])
def test_mla_decode_row_groups(H, tq):
    announce(f"mla decode H={H} tq={tq}")
    m = synth.mla_cache(B=3, H=H, tq=tq, lengths=[5, 300, 999], seed=H + tq)
    assert max_abs(run(m, split_tokens=128), ref(m)) <= BF16_TOL


def test_mla_decode_strided_latent_views():
    # c_kv and k_rope as views of one [B, T, 576] buffer, as a model stores them
    m = synth.mla_cache(B=2, H=16, lengths=[40, 513], seed=9)
    packed = torch.cat([m.c_kv, m.k_rope], dim=-1).cuda()
    o = attn_mla_decode(dev(m.q_nope), dev(m.q_rope), packed[:, :, :512], packed[:, :, 512:], dev(m.w_uk),
                        dev(m.w_uv), cache_off=dev(m.cache_off), split_tokens=256)
    assert max_abs(o, ref(m)) <= BF16_TOL


def test_mla_decode_full_size_B64():
    announce("mla decode full size")
    m = synth.mla_cache(B=64, H=16, seed=0)
    o = run(m)
    batches = [0, 7, 21, 40, 63]
    assert max_abs(o[batches], ref(m, batches)) <= BF16_TOL


def test_mla_decode_rejects_unsupported_width():
    m = synth.mla_cache(B=1, H=4, lengths=[10], rope=32, seed=2)
    with pytest.raises(AttnError, match="kv_rank 512, rope_dim 64"):
        run(m)
