"""Offset-causal attention for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/soc_attn.h`` (``libsoc_attn.so``); this package is the thin binding:

    attn_prefill(q, k, v, cache_off=None, window=0, sink=None, scale=None, block_mask=None, block_list=None)
    attn_decode(q, k, v, cache_off=None, window=0, sink=None, scale=None, split_tokens=0)
    attn_decode_noalloc(q, k, v, cache_off=None, window=0, sink=None, scale=None, split_tokens=0, out=None)
    attn_ring_decode(q, k_new, v_new, k_ring, v_ring, n_seen, sink=None, scale=None)
    attn_mla_decode(q_nope, q_rope, c_kv, k_rope, w_uk, w_uv, cache_off=None)
    attn_dsa_decode(q, k, v, qi, ki, wi, topk, cache_off=None, sink=None)
    attn_block_select(q, k, block_size=128, keep_mean=0.05, keep_radius=0.05, ...)
    attn_block_list_from_mask(mask)
    attn_block_sparse_prefill(q, k, v, cache_off=None, window=0, sink=None, block_size=128, keep_mean=0.05, ...)

PyTorch supplies device memory and the current stream only.  If the library has not
been built, every call raises; there is no fallback path.
"""
from .api import (  # noqa: F401
    AttnError,
    attn_block_list_from_mask,
    attn_block_select,
    attn_block_select_workspace_bytes,
    attn_block_sparse_prefill,
    attn_block_sparse_prefill_workspace_bytes,
    attn_decode,
    attn_decode_noalloc,
    attn_decode_noalloc_max_scratch_bytes,
    attn_decode_workspace_bytes,
    attn_dsa_decode,
    attn_dsa_decode_workspace_bytes,
    attn_mla_decode,
    attn_mla_decode_workspace_bytes,
    attn_prefill,
    attn_ring_decode,
    attn_ring_decode_workspace_bytes,
)
