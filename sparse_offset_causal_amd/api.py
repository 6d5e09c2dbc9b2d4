"""Python binding of the C ABI: argument marshalling only.

Each function takes torch tensors that already live on the GPU, passes their device
pointers, element strides and the current HIP stream to the library, and raises
``AttnError`` on a non-zero return code.  Every step of the computation runs in the
library's HIP kernels; nothing here computes attention.  Output and workspace tensors
are allocated with torch (caller-owned memory) when not supplied.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import AttnMlaShape, AttnShape, AttnStrides


class AttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.ATTN_BF16
    if t.dtype == torch.float32:
        return _lib.ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _check4(name: str, t: torch.Tensor):
    if not isinstance(t, torch.Tensor) or t.dim() != 4:
        raise ValueError(f"{name} must be a 4-D tensor [batch, heads, tokens, head_dim]")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.stride(3) != 1:
        raise ValueError(f"{name} must have a contiguous head_dim axis")


def _strides(t: torch.Tensor) -> AttnStrides:
    return AttnStrides(t.stride(0), t.stride(1), t.stride(2))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(rc: int):
    if rc != 0:
        raise AttnError(rc, _lib.last_error())


def _shape(q: torch.Tensor, k: torch.Tensor) -> AttnShape:
    B, Hq, Tq, d = q.shape
    return AttnShape(B, Hq, k.shape[1], d, Tq, k.shape[2], _dtype_code(q))


def _common(q, k, v, cache_off, sink):
    _check4("q", q)
    _check4("k", k)
    _check4("v", v)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must have the same shape and strides")
    if k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("q and k disagree on batch or head_dim")
    if cache_off is not None and (cache_off.dtype != torch.int32 or not cache_off.is_cuda or
                                  cache_off.numel() != q.shape[0] or not cache_off.is_contiguous()):
        raise ValueError("cache_off must be a contiguous int32 GPU tensor with one entry per sequence")
    if sink is not None and (sink.dtype != torch.float32 or not sink.is_cuda or
                             sink.numel() != q.shape[1] or not sink.is_contiguous()):
        raise ValueError("sink must be a contiguous float32 GPU tensor with one entry per query head")


def _out(q, out):
    if out is None:
        return torch.empty_like(q, memory_format=torch.contiguous_format)
    _check4("out", out)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    return out


def attn_prefill(q, k, v, cache_off=None, window=0, sink=None, scale=None, block_mask=None, block_list=None,
                 block_size=128, out=None):
    """Offset-causal attention of q [B,Hq,Tq,d] against the cache k, v [B,Hkv,Tk,d] (see attn_prefill in
    include/soc_attn.h).  block_mask: uint8 [B, Hq, ceil(Tq/bs), ceil(Tk/bs)], nonzero = kept; or
    block_list: int32 [B, Hq, ceil(Tq/bs), 1 + ceil(Tk/bs)] from attn_block_select."""
    _common(q, k, v, cache_off, sink)
    o = _out(q, out)
    if block_list is not None and (block_list.dtype != torch.int32 or not block_list.is_cuda or
                                   not block_list.is_contiguous()):
        raise ValueError("block_list must be a contiguous int32 GPU tensor")
    if block_mask is not None:
        nqb, nkb = -(-q.shape[2] // block_size), -(-k.shape[2] // block_size)
        if (block_mask.dtype != torch.uint8 or not block_mask.is_cuda or not block_mask.is_contiguous() or
                tuple(block_mask.shape) != (q.shape[0], q.shape[1], nqb, nkb)):
            raise ValueError(f"block_mask must be a contiguous uint8 GPU tensor of shape "
                             f"{(q.shape[0], q.shape[1], nqb, nkb)}")
    lib = _lib.load()
    shape = _shape(q, k)
    rc = lib.attn_prefill(shape, q.data_ptr(), _strides(q), k.data_ptr(), v.data_ptr(), _strides(k),
                          o.data_ptr(), _strides(o), _ptr(cache_off), int(window), _ptr(sink),
                          float(scale or 0.0), _ptr(block_mask), _ptr(block_list), int(block_size), _stream())
    _check(rc)
    return o


def attn_decode_workspace_bytes(q, k, split_tokens=0) -> int:
    return int(_lib.load().attn_decode_workspace_bytes(_shape(q, k), int(split_tokens)))


def attn_decode(q, k, v, cache_off=None, window=0, sink=None, scale=None, split_tokens=0, workspace=None,
                out=None):
    """Split-KV decode (see attn_decode in include/soc_attn.h).  workspace: a uint8 GPU tensor of at least
    attn_decode_workspace_bytes() bytes; allocated here when omitted."""
    _common(q, k, v, cache_off, sink)
    o = _out(q, out)
    lib = _lib.load()
    shape = _shape(q, k)
    need = int(lib.attn_decode_workspace_bytes(shape, int(split_tokens)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rc = lib.attn_decode(shape, q.data_ptr(), _strides(q), k.data_ptr(), v.data_ptr(), _strides(k),
                         o.data_ptr(), _strides(o), _ptr(cache_off), int(window), _ptr(sink), float(scale or 0.0),
                         workspace.data_ptr(), workspace.numel() * workspace.element_size(), int(split_tokens),
                         _stream())
    _check(rc)
    return o


def attn_decode_noalloc_max_scratch_bytes() -> int:
    return int(_lib.load().attn_decode_noalloc_max_scratch_bytes())


def attn_decode_noalloc(q, k, v, cache_off=None, window=0, sink=None, scale=None, split_tokens=0, out=None):
    """attn_decode without a workspace: the library's per-GPU scratch holds the partials (see
    attn_decode_noalloc in include/soc_attn.h).  Pass ``out`` to allocate nothing at all."""
    _common(q, k, v, cache_off, sink)
    o = _out(q, out)
    lib = _lib.load()
    rc = lib.attn_decode_noalloc(_shape(q, k), q.data_ptr(), _strides(q), k.data_ptr(), v.data_ptr(), _strides(k),
                                 o.data_ptr(), _strides(o), _ptr(cache_off), int(window), _ptr(sink),
                                 float(scale or 0.0), int(split_tokens), _stream())
    _check(rc)
    return o


def attn_ring_decode_workspace_bytes(q, k_ring, split_tokens=0) -> int:
    return int(_lib.load().attn_ring_decode_workspace_bytes(_shape(q, k_ring), int(split_tokens)))


def attn_ring_decode(q, k_new, v_new, k_ring, v_ring, n_seen, sink=None, scale=None, split_tokens=0,
                     workspace=None, out=None):
    """One sliding-window decode step over a W-slot ring cache (see attn_ring_decode in
    include/soc_attn.h): writes k_new / v_new [B,Hkv,1,d] into slot n_seen[b] % W of k_ring / v_ring
    [B,Hkv,W,d] (in place) and returns the attention of q [B,Hq,1,d] over the filled slots.  n_seen is
    an int32 GPU tensor [B] the caller advances after the step."""
    _common(q, k_ring, v_ring, None, sink)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _check4(name, t)
        if t.dtype != q.dtype or t.shape != (k_ring.shape[0], k_ring.shape[1], 1, k_ring.shape[3]):
            raise ValueError(f"{name} must be [B, Hkv, 1, d] in the ring's dtype")
    if k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new must share strides")
    if (n_seen.dtype != torch.int32 or not n_seen.is_cuda or n_seen.numel() != q.shape[0] or
            not n_seen.is_contiguous()):
        raise ValueError("n_seen must be a contiguous int32 GPU tensor with one entry per sequence")
    o = _out(q, out)
    lib = _lib.load()
    shape = _shape(q, k_ring)
    need = int(lib.attn_ring_decode_workspace_bytes(shape, int(split_tokens)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rc = lib.attn_ring_decode(shape, q.data_ptr(), _strides(q), k_new.data_ptr(), v_new.data_ptr(), _strides(k_new),
                              k_ring.data_ptr(), v_ring.data_ptr(), _strides(k_ring), o.data_ptr(), _strides(o),
                              n_seen.data_ptr(), _ptr(sink), float(scale or 0.0), workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), int(split_tokens), _stream())
    _check(rc)
    return o


def _mla_shape(q_nope, q_rope, c_kv, k_rope, w_uv):
    B, H, Tq, dn = q_nope.shape
    return AttnMlaShape(B, H, Tq, c_kv.shape[1], c_kv.shape[2], q_rope.shape[3], dn, w_uv.shape[2],
                        _dtype_code(q_nope))


def attn_mla_decode_workspace_bytes(q_nope, q_rope, c_kv, k_rope, w_uv, split_tokens=0) -> int:
    return int(_lib.load().attn_mla_decode_workspace_bytes(_mla_shape(q_nope, q_rope, c_kv, k_rope, w_uv),
                                                           int(split_tokens)))


def attn_mla_decode(q_nope, q_rope, c_kv, k_rope, w_uk, w_uv, cache_off=None, scale=None, split_tokens=0,
                    workspace=None, out=None):
    """Multi-head latent attention decode in absorbed form (see attn_mla_decode in include/soc_attn.h).
    q_nope [B,H,Tq,128], q_rope [B,H,Tq,64], c_kv [B,Tk,512], k_rope [B,Tk,64] (token axis strided,
    last axis contiguous), w_uk [H,512,128], w_uv [H,512,128] contiguous; returns o [B,H,Tq,128]."""
    _check4("q_nope", q_nope)
    _check4("q_rope", q_rope)
    for name, t in (("c_kv", c_kv), ("k_rope", k_rope)):
        if t.dim() != 3 or not t.is_cuda or t.stride(2) != 1:
            raise ValueError(f"{name} must be a 3-D GPU tensor [batch, tokens, width] with a contiguous last axis")
    for name, t in (("w_uk", w_uk), ("w_uv", w_uv)):
        if t.dim() != 3 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 3-D GPU tensor [heads, kv_rank, width]")
    if len({t.dtype for t in (q_nope, q_rope, c_kv, k_rope, w_uk, w_uv)}) != 1:
        raise ValueError("all MLA inputs must share one dtype")
    if cache_off is not None and (cache_off.dtype != torch.int32 or not cache_off.is_cuda or
                                  cache_off.numel() != q_nope.shape[0] or not cache_off.is_contiguous()):
        raise ValueError("cache_off must be a contiguous int32 GPU tensor with one entry per sequence")
    B, H, Tq, _ = q_nope.shape
    if out is None:
        out = torch.empty((B, H, Tq, w_uv.shape[2]), dtype=q_nope.dtype, device=q_nope.device)
    lib = _lib.load()
    shape = _mla_shape(q_nope, q_rope, c_kv, k_rope, w_uv)
    need = int(lib.attn_mla_decode_workspace_bytes(shape, int(split_tokens)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_nope.device)
    bt = lambda t: AttnStrides(t.stride(0), 0, t.stride(1))
    rc = lib.attn_mla_decode(shape, q_nope.data_ptr(), _strides(q_nope), q_rope.data_ptr(), _strides(q_rope),
                             c_kv.data_ptr(), bt(c_kv), k_rope.data_ptr(), bt(k_rope), w_uk.data_ptr(),
                             w_uv.data_ptr(), out.data_ptr(), _strides(out), _ptr(cache_off), float(scale or 0.0),
                             workspace.data_ptr(), workspace.numel() * workspace.element_size(), int(split_tokens),
                             _stream())
    _check(rc)
    return out


def attn_dsa_decode_workspace_bytes(q, k, topk, split_tokens=0) -> int:
    return int(_lib.load().attn_dsa_decode_workspace_bytes(_shape(q, k), int(topk), int(split_tokens)))


def attn_dsa_decode(q, k, v, qi, ki, wi, topk, cache_off=None, sink=None, scale=None, split_tokens=0,
                    want_kept=False, workspace=None, out=None):
    """Token top-k sparse attention decode (see attn_dsa_decode in include/soc_attn.h): q [B,Hq,Tq,128],
    k, v [B,Hkv,Tk,128], qi [B,Hi,Tq,128], ki [B,Tk,128] (token axis strided), wi float32 [B,Hi,Tq].
    Returns o, or (o, kept_list [B,Tq,topk], kept_count [B,Tq]) with want_kept."""
    _common(q, k, v, cache_off, sink)
    _check4("qi", qi)
    if ki.dim() != 3 or not ki.is_cuda or ki.stride(2) != 1 or ki.dtype != q.dtype:
        raise ValueError("ki must be a 3-D GPU tensor [batch, tokens, 128] in q's dtype with a contiguous last axis")
    if wi.dtype != torch.float32 or not wi.is_cuda or not wi.is_contiguous() or wi.shape != (q.shape[0], qi.shape[1], q.shape[2]):
        raise ValueError("wi must be a contiguous float32 GPU tensor [batch, index_heads, tq]")
    o = _out(q, out)
    lib = _lib.load()
    shape = _shape(q, k)
    need = int(lib.attn_dsa_decode_workspace_bytes(shape, int(topk), int(split_tokens)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    kl = kc = None
    if want_kept:
        kl = torch.empty((q.shape[0], q.shape[2], int(topk)), dtype=torch.int32, device=q.device)
        kc = torch.empty((q.shape[0], q.shape[2]), dtype=torch.int32, device=q.device)
    rc = lib.attn_dsa_decode(shape, q.data_ptr(), _strides(q), k.data_ptr(), v.data_ptr(), _strides(k), o.data_ptr(),
                             _strides(o), _ptr(cache_off), _ptr(sink), float(scale or 0.0), qi.data_ptr(),
                             _strides(qi), ki.data_ptr(), AttnStrides(ki.stride(0), 0, ki.stride(1)), wi.data_ptr(),
                             int(qi.shape[1]), int(topk), _ptr(kl), _ptr(kc), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), int(split_tokens), _stream())
    _check(rc)
    return (o, kl, kc) if want_kept else o


def attn_block_select_workspace_bytes(q, k, block_size=128) -> int:
    return int(_lib.load().attn_block_select_workspace_bytes(_shape(q, k), int(block_size)))


def attn_block_select(q, k, block_size=128, cache_off=None, window=0, keep_mean=0.05, keep_radius=0.05,
                      tau_mean=None, tau_radius=None, want_list=True, workspace=None):
    """Block mask from the mean-centroid branch OR the max-radius branch (see attn_block_select in
    include/soc_attn.h).  Returns dict(mask, list, tau_mean, tau_radius); negative keep fractions read
    the caller's tau_mean / tau_radius (float64 GPU tensors [B,Hq] / [B,Hkv])."""
    _check4("q", q)
    _check4("k", k)
    if k.dtype != q.dtype:
        raise ValueError("q and k must share one dtype")
    if cache_off is not None and (cache_off.dtype != torch.int32 or not cache_off.is_cuda or
                                  cache_off.numel() != q.shape[0]):
        raise ValueError("cache_off must be an int32 GPU tensor with one entry per sequence")
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    nqb, nkb = -(-Tq // block_size), -(-Tk // block_size)
    dev = q.device
    if tau_mean is None:
        if keep_mean < 0:
            raise ValueError("keep_mean < 0 needs tau_mean")
        tau_mean = torch.empty((B, Hq), dtype=torch.float64, device=dev)
    if tau_radius is None:
        if keep_radius < 0:
            raise ValueError("keep_radius < 0 needs tau_radius")
        tau_radius = torch.empty((B, Hkv), dtype=torch.float64, device=dev)
    for name, t, shp in (("tau_mean", tau_mean, (B, Hq)), ("tau_radius", tau_radius, (B, Hkv))):
        if t.dtype != torch.float64 or not t.is_cuda or tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float64 GPU tensor of shape {shp}")
    mask = torch.empty((B, Hq, nqb, nkb), dtype=torch.uint8, device=dev)
    lst = torch.empty((B, Hq, nqb, 1 + nkb), dtype=torch.int32, device=dev) if want_list else None
    lib = _lib.load()
    shape = _shape(q, k)
    need = int(lib.attn_block_select_workspace_bytes(shape, int(block_size)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib.attn_block_select(shape, q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), _ptr(cache_off),
                               int(window), int(block_size), float(keep_mean), float(keep_radius),
                               tau_mean.data_ptr(), tau_radius.data_ptr(), mask.data_ptr(), _ptr(lst),
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream())
    _check(rc)
    return dict(mask=mask, list=lst, tau_mean=tau_mean, tau_radius=tau_radius)


def attn_block_sparse_prefill_workspace_bytes(q, k, block_size=128) -> int:
    return int(_lib.load().attn_block_sparse_prefill_workspace_bytes(_shape(q, k), int(block_size)))


def attn_block_sparse_prefill(q, k, v, cache_off=None, window=0, sink=None, scale=None, block_size=128,
                              keep_mean=0.05, keep_radius=0.05, tau_mean=None, tau_radius=None, want_mask=False,
                              workspace=None, out=None):
    """Block selection and block-sparse prefill in one call (see attn_block_sparse_prefill in
    include/soc_attn.h).  Returns o, or (o, dict(mask, tau_mean, tau_radius)) with want_mask."""
    _common(q, k, v, cache_off, sink)
    o = _out(q, out)
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    dev = q.device
    if tau_mean is None:
        if keep_mean < 0:
            raise ValueError("keep_mean < 0 needs tau_mean")
        tau_mean = torch.empty((B, Hq), dtype=torch.float64, device=dev)
    if tau_radius is None:
        if keep_radius < 0:
            raise ValueError("keep_radius < 0 needs tau_radius")
        tau_radius = torch.empty((B, Hkv), dtype=torch.float64, device=dev)
    for name, t, shp in (("tau_mean", tau_mean, (B, Hq)), ("tau_radius", tau_radius, (B, Hkv))):
        if t.dtype != torch.float64 or not t.is_cuda or tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float64 GPU tensor of shape {shp}")
    mask = None
    if want_mask:
        mask = torch.empty((B, Hq, -(-Tq // block_size), -(-Tk // block_size)), dtype=torch.uint8, device=dev)
    lib = _lib.load()
    shape = _shape(q, k)
    need = int(lib.attn_block_sparse_prefill_workspace_bytes(shape, int(block_size)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib.attn_block_sparse_prefill(shape, q.data_ptr(), _strides(q), k.data_ptr(), v.data_ptr(), _strides(k),
                                       o.data_ptr(), _strides(o), _ptr(cache_off), int(window), _ptr(sink),
                                       float(scale or 0.0), int(block_size), float(keep_mean), float(keep_radius),
                                       tau_mean.data_ptr(), tau_radius.data_ptr(), _ptr(mask), workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), _stream())
    _check(rc)
    return (o, dict(mask=mask, tau_mean=tau_mean, tau_radius=tau_radius)) if want_mask else o


def attn_block_list_from_mask(mask):
    """Kept-block list (int32 [..., 1 + n_kb]) from a uint8 GPU block mask [..., n_kb]."""
    if mask.dtype != torch.uint8 or not mask.is_cuda or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous uint8 GPU tensor")
    n_kb = mask.shape[-1]
    rows = mask.numel() // n_kb
    lst = torch.empty(mask.shape[:-1] + (1 + n_kb,), dtype=torch.int32, device=mask.device)
    _check(_lib.load().attn_block_list_from_mask(rows, n_kb, mask.data_ptr(), lst.data_ptr(), _stream()))
    return lst
