"""Seeded synthetic inputs for the offset-causal attention workloads.

This module holds random draws and workload recipes only (shapes, seeds, cache
lengths, planted keys).  It contains none of the attention arithmetic, so the
oracle side and the GPU side can both read from it without sharing any of the
method's code.

Every tensor is drawn on the CPU as float32 N(0, 1) from its own
``torch.Generator`` and then rounded to the run dtype (bf16 by round-to-nearest-even,
or kept as f32).  Per-tensor seeds follow one base seed ``s``:

    q = s, k = s+1, v = s+2, sink = s+3, cache lengths = s+4, planted keys = s+5.

Workload shapes follow the pages' examples: head dim 16 with 8 query heads and
2 KV heads over 40 tokens (sotaaz.com/post/attention-in-code, section 1 on
MHA/MQA/GQA), a window of 8 (same page, section 2 on the ring buffer), and
long-context prefill with an important key hidden inside a block of ordinary
keys (patty.io review of RBS-Attention, section on mean dilution).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

SEED_Q, SEED_K, SEED_V, SEED_SINK, SEED_LEN, SEED_OUTLIER = 0, 1, 2, 3, 4, 5


def normal(shape, seed: int, dtype=torch.float32) -> torch.Tensor:
    """float32 N(0,1) draw from a fresh generator seeded with ``seed``, cast to ``dtype``."""
    g = torch.Generator().manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


@dataclass
class Workload:
    """One attention call's inputs.

    q: [B, Hq, Tq, d]; k, v: [B, Hkv, Tk, d] where Tk is the number of cache rows
    addressable per sequence.  ``cache_off`` (int32 [B]) gives each sequence's cache
    offset; None means offset = Tk - Tq for every sequence.  ``window`` <= 0 means no
    window.  ``sink`` is float32 [Hq] or None.  ``scale`` None means 1/sqrt(d).
    """

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cache_off: Optional[torch.Tensor] = None
    window: int = 0
    sink: Optional[torch.Tensor] = None
    scale: Optional[float] = None
    block_size: int = 0
    keep_mean: float = 0.0
    keep_radius: float = 0.0
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, Hq, Tq, d = self.q.shape
        return dict(batch=B, n_heads=Hq, n_kv=self.k.shape[1], head_dim=d, tq=Tq, tk=self.k.shape[2])


def attention_inputs(B, Hq, Hkv, Tq, Tk, d, dtype, seed=0, with_sink=False, window=0,
                     cache_off=None, name="custom") -> Workload:
    """Plain N(0,1) q/k/v (and optionally sink) with the standard per-tensor seeds."""
    q = normal((B, Hq, Tq, d), seed + SEED_Q, dtype)
    k = normal((B, Hkv, Tk, d), seed + SEED_K, dtype)
    v = normal((B, Hkv, Tk, d), seed + SEED_V, dtype)
    sink = normal((Hq,), seed + SEED_SINK) if with_sink else None
    off = None if cache_off is None else torch.as_tensor(cache_off, dtype=torch.int32)
    return Workload(name, q, k, v, cache_off=off, window=window, sink=sink)


def tiny(seed=0, with_sink=False, window=0) -> Workload:
    """Batch 1, 8 query heads, 2 KV heads, head dim 16, T = 40, float32."""
    return attention_inputs(1, 8, 2, 40, 40, 16, torch.float32, seed, with_sink, window,
                            name="tiny_f32_T40")


def causal_prefill(T=8192, Hq=32, Hkv=8, d=128, seed=0) -> Workload:
    """Causal prefill at cache offset 0, bf16, scale 1/sqrt(d)."""
    w = attention_inputs(1, Hq, Hkv, T, T, d, torch.bfloat16, seed,
                         name=f"causal_prefill_bf16_T{T}_{Hq}q{Hkv}kv_d{d}")
    w.cache_off = torch.zeros(1, dtype=torch.int32)
    w.scale = 1.0 / math.sqrt(d)
    return w


def window_sink_prefill(T=32768, W=1024, Hq=32, Hkv=8, d=128, seed=0) -> Workload:
    """Sliding-window causal prefill with one N(0,1) sink logit per query head, bf16."""
    w = attention_inputs(1, Hq, Hkv, T, T, d, torch.bfloat16, seed, with_sink=True, window=W,
                         name=f"window_sink_prefill_bf16_T{T}_W{W}_{Hq}q{Hkv}kv_d{d}")
    w.cache_off = torch.zeros(1, dtype=torch.int32)
    return w


def cache_lengths(B, lo, hi, seed=0) -> torch.Tensor:
    """Per-sequence cached token counts, uniform integers in [lo, hi] inclusive."""
    g = torch.Generator().manual_seed(seed + SEED_LEN)
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


@dataclass
class DecodeCache:
    """A KV cache holding L_b tokens per sequence plus room for ``chunk`` new ones.

    k, v: [B, Hkv, cap, d] with cap = max(L) + chunk; rows at or beyond L_b + chunk are
    zero (never addressed).  q_decode: [B, Hq, 1, d] (the new token, whose K/V sit at row
    L_b).  q_chunk: [B, Hq, chunk, d] (a chunk whose K/V sit at rows L_b .. L_b+chunk-1).
    """

    lengths: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    q_decode: torch.Tensor
    q_chunk: torch.Tensor
    chunk: int

    def decode(self) -> Workload:
        return Workload("decode", self.q_decode, self.k, self.v, cache_off=self.lengths.clone())

    def prefill_chunk(self) -> Workload:
        return Workload("chunk", self.q_chunk, self.k, self.v, cache_off=self.lengths.clone())


def decode_cache(B=64, lo=1024, hi=32768, chunk=512, Hq=32, Hkv=8, d=128, seed=0,
                 dtype=torch.bfloat16) -> DecodeCache:
    """Cache lengths uniform in [lo, hi]; valid rows of k/v drawn N(0,1) sequence by sequence."""
    L = cache_lengths(B, lo, hi, seed)
    cap = int(L.max()) + chunk
    k = torch.zeros((B, Hkv, cap, d), dtype=dtype)
    v = torch.zeros((B, Hkv, cap, d), dtype=dtype)
    gk = torch.Generator().manual_seed(seed + SEED_K)
    gv = torch.Generator().manual_seed(seed + SEED_V)
    for b in range(B):
        n = int(L[b]) + chunk
        k[b, :, :n] = torch.randn((Hkv, n, d), generator=gk).to(dtype)
        v[b, :, :n] = torch.randn((Hkv, n, d), generator=gv).to(dtype)
    q_dec = normal((B, Hq, 1, d), seed + SEED_Q, dtype)
    q_chunk = normal((B, Hq, chunk, d), seed + SEED_Q + 100, dtype)
    return DecodeCache(L, k, v, q_dec, q_chunk, chunk)


def block_sparse_prefill(T=65536, BS=128, Hq=32, Hkv=8, d=128, frac=0.05, norm_mult=6.0,
                         keep_mean=0.05, keep_radius=0.05, seed=0) -> Workload:
    """Long causal prefill with planted outlier keys.

    q, v ~ N(0,1).  k ~ N(0,1) except that, for every KV head, round(frac * nb) key blocks
    (nb = T / BS, chosen without replacement) each get one key replaced: at a random slot
    of the block, the key becomes ``norm_mult * sqrt(d)`` times the unit vector of the
    mean of a random query block qb >= kb, the mean taken over the group's query heads and
    the block's rows (bf16 values, computed in float64).  Planted positions are returned
    in ``meta['planted']`` as (kv_head, key_block, slot, query_block) rows.
    """
    w = attention_inputs(1, Hq, Hkv, T, T, d, torch.bfloat16, seed,
                         name=f"block_sparse_prefill_bf16_T{T}_BS{BS}_{Hq}q{Hkv}kv_d{d}")
    w.cache_off = torch.zeros(1, dtype=torch.int32)
    nb = T // BS
    g_heads = Hq // Hkv
    n_plant = int(math.floor(frac * nb + 0.5))
    gen = torch.Generator().manual_seed(seed + SEED_OUTLIER)
    planted = []
    for kvh in range(Hkv):
        blocks = torch.randperm(nb, generator=gen)[:n_plant].sort().values
        for kb in blocks.tolist():
            slot = int(torch.randint(0, BS, (1,), generator=gen))
            qb = int(torch.randint(kb, nb, (1,), generator=gen))
            rows = w.q[0, kvh * g_heads:(kvh + 1) * g_heads, qb * BS:(qb + 1) * BS, :]
            mean = rows.to(torch.float64).reshape(-1, d).mean(0)
            key = norm_mult * math.sqrt(d) * mean / mean.norm()
            w.k[0, kvh, kb * BS + slot] = key.to(w.k.dtype)
            planted.append((kvh, kb, slot, qb))
    w.block_size = BS
    w.keep_mean = keep_mean
    w.keep_radius = keep_radius
    w.meta["planted"] = planted
    return w


@dataclass
class RingState:
    """A W-slot ring cache per (sequence, KV head) and the per-sequence count of tokens
    already written (n_seen).  Slots a sequence has not written yet (slot >= n_seen when
    n_seen < W) hold large stale values that a correct reader never touches."""

    k: torch.Tensor       # [B, Hkv, W, d]
    v: torch.Tensor       # [B, Hkv, W, d]
    n_seen: torch.Tensor  # [B] int32
    sink: torch.Tensor    # [Hq] float32


def ring_state(B=64, Hq=32, Hkv=8, d=128, W=1024, n_lo=0, n_hi=4096, seed=0, dtype=torch.bfloat16,
               stale=1.0e4, n_seen=None) -> RingState:
    """Ring contents N(0,1); n_seen uniform integers in [n_lo, n_hi] (or the given list);
    sink N(0,1) per head."""
    k = normal((B, Hkv, W, d), seed + SEED_K, torch.float32)
    v = normal((B, Hkv, W, d), seed + SEED_V, torch.float32)
    n = cache_lengths(B, n_lo, n_hi, seed) if n_seen is None else torch.tensor(n_seen, dtype=torch.int32)
    for b in range(B):
        if int(n[b]) < W:
            k[b, :, int(n[b]):] = stale
            v[b, :, int(n[b]):] = stale
    sink = normal((Hq,), seed + SEED_SINK)
    return RingState(k.to(dtype), v.to(dtype), n, sink)


def ring_step(B, Hq, Hkv, d, step, seed=0, dtype=torch.bfloat16):
    """One decode step's inputs: q [B, Hq, 1, d] and the new token's k, v [B, Hkv, 1, d]."""
    base = seed + 1000 + 10 * step
    return (normal((B, Hq, 1, d), base + SEED_Q, dtype), normal((B, Hkv, 1, d), base + SEED_K, dtype),
            normal((B, Hkv, 1, d), base + SEED_V, dtype))


@dataclass
class MlaCache:
    """A latent KV cache (multi-head latent attention) with random projection weights.

    c_kv [B, cap, 512], k_rope [B, cap, 64]: rows 0..L_b hold the cached tokens plus the
    step's own token(s); q_nope [B, H, tq, 128], q_rope [B, H, tq, 64]; w_uk, w_uv
    [H, 512, 128] drawn N(0, 1/128) and N(0, 1/512) so that folded queries and outputs stay
    near unit scale; cache_off = L_b (the step's tokens sit at rows L_b .. L_b + tq - 1)."""

    q_nope: torch.Tensor
    q_rope: torch.Tensor
    c_kv: torch.Tensor
    k_rope: torch.Tensor
    w_uk: torch.Tensor
    w_uv: torch.Tensor
    cache_off: torch.Tensor


def mla_cache(B=64, H=16, lengths=None, lo=1024, hi=32768, tq=1, rank=512, rope=64, nope=128, dv=128, seed=0,
              dtype=torch.bfloat16) -> MlaCache:
    L = cache_lengths(B, lo, hi, seed) if lengths is None else torch.tensor(lengths, dtype=torch.int32)
    cap = int(L.max()) + tq
    c_kv = torch.zeros((B, cap, rank), dtype=dtype)
    k_rope = torch.zeros((B, cap, rope), dtype=dtype)
    gk = torch.Generator().manual_seed(seed + SEED_K)
    for b in range(B):
        n = int(L[b]) + tq
        c_kv[b, :n] = torch.randn((n, rank), generator=gk).to(dtype)
        k_rope[b, :n] = torch.randn((n, rope), generator=gk).to(dtype)
    q_nope = normal((B, H, tq, nope), seed + SEED_Q, dtype)
    q_rope = normal((B, H, tq, rope), seed + SEED_Q + 100, dtype)
    w_uk = (normal((H, rank, nope), seed + SEED_V) / math.sqrt(nope)).to(dtype)
    w_uv = (normal((H, rank, dv), seed + SEED_V + 100) / math.sqrt(rank)).to(dtype)
    return MlaCache(q_nope, q_rope, c_kv, k_rope, w_uk, w_uv, L)


@dataclass
class DsaInputs:
    """A KV cache for token top-k sparse decode: q [B, Hq, tq, d], k, v [B, Hkv, cap, d]
    (rows 0..L_b + tq - 1 drawn, the rest zero), the indexer's qi [B, Hi, tq, di] and
    ki [B, cap, di] (N(0,1)) and head weights wi [B, Hi, tq] (N(0, 1/Hi)), cache_off = L_b."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    qi: torch.Tensor
    ki: torch.Tensor
    wi: torch.Tensor
    sink: torch.Tensor
    cache_off: torch.Tensor


def dsa_inputs(B=64, Hq=32, Hkv=8, tq=1, lengths=None, lo=1024, hi=32768, Hi=64, d=128, di=128, seed=0,
               dtype=torch.bfloat16) -> DsaInputs:
    L = cache_lengths(B, lo, hi, seed) if lengths is None else torch.tensor(lengths, dtype=torch.int32)
    cap = int(L.max()) + tq
    k = torch.zeros((B, Hkv, cap, d), dtype=dtype)
    v = torch.zeros((B, Hkv, cap, d), dtype=dtype)
    ki = torch.zeros((B, cap, di), dtype=dtype)
    gk = torch.Generator().manual_seed(seed + SEED_K)
    gv = torch.Generator().manual_seed(seed + SEED_V)
    for b in range(B):
        n = int(L[b]) + tq
        k[b, :, :n] = torch.randn((Hkv, n, d), generator=gk).to(dtype)
        v[b, :, :n] = torch.randn((Hkv, n, d), generator=gv).to(dtype)
        ki[b, :n] = torch.randn((n, di), generator=gk).to(dtype)
    q = normal((B, Hq, tq, d), seed + SEED_Q, dtype)
    qi = normal((B, Hi, tq, di), seed + SEED_Q + 100, dtype)
    wi = normal((B, Hi, tq), seed + SEED_Q + 200) / math.sqrt(Hi)
    sink = normal((Hq,), seed + SEED_SINK)
    return DsaInputs(q, k, v, qi, ki, wi, sink, L)
