"""attn_decode_noalloc (the decode entry point that allocates nothing; its partials live in
the library's per-GPU scratch array) against attn_decode with a caller workspace, through
the C ABI.  Two calls in a row, the second smaller than the first, so that the second runs
on scratch the first left behind; outputs must equal attn_decode's bit for bit (the same
kernels with the same split) and the float64 oracle within the bf16 bound."""
import pytest
import torch

import synth
from oracle import attend
from sparse_offset_causal_amd import (AttnError, attn_decode, attn_decode_noalloc, attn_decode_noalloc_max_scratch_bytes,
                                      attn_decode_workspace_bytes)
from tests.gpu_helpers import BF16_TOL, announce, dev, max_abs, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def one_call(w, window, split):
    q, k, v, off, sink = dev(w.q), dev(w.k), dev(w.v), dev(w.cache_off), dev(w.sink)
    out = torch.empty_like(q)
    got = attn_decode_noalloc(q, k, v, cache_off=off, window=window, sink=sink, split_tokens=split, out=out)
    want = attn_decode(q, k, v, cache_off=off, window=window, sink=sink, split_tokens=split)
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got, want)
    ref = attend(w.q, w.k, w.v, cache_off=w.cache_off, window=window, sink=w.sink)
    assert max_abs(got, ref) <= BF16_TOL


def test_noalloc_decode_matches_workspace_decode_twice():
    announce("no-allocation decode: two calls, the second smaller")
    big = synth.attention_inputs(6, 32, 8, 2, 5000, 128, torch.bfloat16, seed=71, with_sink=True,
                                 cache_off=[4998, 17, 3000, 1024, 2047, 4500])
    small = synth.attention_inputs(2, 8, 2, 1, 700, 128, torch.bfloat16, seed=72, with_sink=True,
                                   cache_off=[699, 5])
    one_call(big, 0, 256)
    one_call(small, 300, 0)


def test_noalloc_decode_rejects_shapes_beyond_its_scratch():
    cap = attn_decode_noalloc_max_scratch_bytes()
    assert cap == 32 << 20
    # batch 64, 32 heads, 8 query rows each, 20000-key cache at 256-key splits needs far more
    q = torch.empty((64, 32, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((64, 8, 20000, 128), dtype=torch.bfloat16, device="cuda")
    assert attn_decode_workspace_bytes(q, k, 256) > cap
    with pytest.raises(AttnError, match="scratch"):
        attn_decode_noalloc(q, k, k, split_tokens=256)
