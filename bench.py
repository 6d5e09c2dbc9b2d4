"""Benchmark: offset-causal attention on one MI355X.

One step = one call of the hot path on one batch of synthetic input.  The headline
``value`` is causal prefill throughput (TFLOP/s of algorithmic work) on the workload
"batch 1, 32 query / 8 KV heads, head_dim 128, Tq = Tk = 8192, bf16".  The same JSON line
also carries, under ``also``, the other workloads of the path measured the same way:
sliding-window prefill with sinks (T = 32768, W = 1024), KV-cache decode (batch 64, cache
lengths uniform in [1024, 32768]; decode KV-read GB/s), a 512-token chunk appended at each
sequence's cache offset, sliding-window decode over W = 1024-slot ring caches with the
step's K/V appended (batch 64), multi-head latent attention decode in absorbed form
(batch 64, 16 heads, 576 numbers per cached token), token top-k sparse decode with its
indexer (batch 64, top 2048), and block-sparse prefill (T = 65536, block 128) with its
block selection.

Algorithmic work: prefill flops = 4 * head_dim * sum over heads of the allowed (row, key)
pairs (QK^T and PV, 2 flops per multiply-add; masked halves of tiles and the softmax are not
counted).  Decode bytes = K and V rows each sequence must read (2 * n_kv * Tk_b * d * 2 B)
plus q and o.  Inputs are resident in HBM before timing starts.

Timing: ``warmup`` untimed steps, then exactly ``steps`` steps between two device
synchronisations, with one pair of HIP events on the stream the kernels run on bracketing
the timed steps (GPU time per step = their elapsed time / steps).  Per-call event timings
(an event pair around each call, which adds a few microseconds of queue serialisation per
call) are taken on a few extra calls after the timed region and reported as
``call_ms_median`` / ``call_ms_min``.  ``cpu_baseline`` times the float64 oracle on the host
on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from sparse_offset_causal_amd import (attn_block_select, attn_block_select_workspace_bytes,  # noqa: E402
                                      attn_block_sparse_prefill, attn_decode, attn_decode_workspace_bytes,
                                      attn_dsa_decode, attn_dsa_decode_workspace_bytes, attn_mla_decode, attn_mla_decode_workspace_bytes, attn_prefill,
                                      attn_ring_decode, attn_ring_decode_workspace_bytes)

METRIC = "prefill TFLOP/s + decode KV-read GB/s, offset-causal GQA attention, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E


# ------------------------------------------------------------------ algorithmic work
def allowed_pairs(tq: int, tkb: int, window: int) -> int:
    """(row, key) pairs the rule allows for one head: row r at pos = tkb - tq + r sees
    keys max(0, pos - W + 1) .. pos."""
    pos = np.arange(tkb - tq, tkb, dtype=np.int64)
    lo = np.maximum(0, pos - window + 1) if window > 0 else np.zeros_like(pos)
    return int((pos - lo + 1).sum())


def prefill_flops(Hq, d, pairs_per_head_total):
    return 4.0 * d * Hq * pairs_per_head_total


def block_pairs(bs: int, qb: int, kb: int) -> int:
    """Allowed pairs of a kept (query block, key block) at offset 0 without a window."""
    if kb < qb:
        return bs * bs
    if kb == qb:
        return bs * (bs + 1) // 2
    return 0


# ------------------------------------------------------------------ timing
class Timer:
    """Times `steps` calls of fn between synchronisations.  The timed region holds only the
    calls: the wall clock and one pair of HIP events on the launch stream bracket it (the
    events give the mean GPU time per step).  Per-call event timings, which put an event pair
    around every call and so perturb short steps, are taken afterwards on a few extra calls."""

    def __init__(self, fn, steps, warmup):
        self.fn, self.steps, self.warmup = fn, steps, warmup

    def run(self):
        for _ in range(self.warmup):
            self.fn()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(self.steps):
            self.fn()
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms = start.elapsed_time(end) / self.steps
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(min(self.steps, 10))]
        for s, e in ev:
            s.record(stream)
            self.fn()
            e.record(stream)
        torch.cuda.synchronize()
        per = [s.elapsed_time(e) for s, e in ev]  # ms
        return dict(wall_s=wall, ms_per_step=wall * 1e3 / self.steps, gpu_ms_per_step=gpu_ms,
                    call_ms_median=float(np.median(per)), call_ms_min=float(np.min(per)))


class OracleClock:
    """Times the float64 oracle on the host on a bounded sample of a workload: `units` are
    callables (one sampled piece of the workload each) run in order until `budget_s` has
    passed; `work` gives each piece's algorithmic work (flops or bytes, as the GPU line
    counts them).  Reported as a rate in the GPU line's unit, with the host threads used."""

    enabled = True
    cores = 1

    @classmethod
    def run(cls, units, work, scale, unit, what, budget_s=3.0):
        if not cls.enabled:
            return None
        done, w, t0 = 0, 0.0, time.perf_counter()
        for fn, wk in zip(units, work):
            fn()
            done += 1
            w += wk
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": w / dt / scale, "unit": unit, "cores": cls.cores, "kind": "oracle",
                "sample": f"{done} {what} (float64 numpy/BLAS), {dt:.1f} s"}


def to_dev(w):
    f = lambda t: None if t is None else t.to("cuda", non_blocking=False)
    return f(w.q), f(w.k), f(w.v), f(w.cache_off), f(w.sink)


# ------------------------------------------------------------------ workloads
def bench_causal_prefill(steps, warmup, T=8192):
    w = synth.causal_prefill(T=T)
    q, k, v, off, _ = to_dev(w)
    out = torch.empty_like(q)
    fn = lambda: attn_prefill(q, k, v, cache_off=off, scale=w.scale, out=out)
    r = Timer(fn, steps, warmup).run()
    flops = prefill_flops(32, 128, allowed_pairs(T, T, 0))
    r.update(workload=w.name, flops_per_step=flops, value=flops / (r["ms_per_step"] * 1e-3) / 1e12,
             kernel_tflops=flops / (r["gpu_ms_per_step"] * 1e-3) / 1e12, unit="TFLOP/s")
    return r, w


def bench_window_sink(steps, warmup, T=32768, W=1024):
    w = synth.window_sink_prefill(T=T, W=W)
    q, k, v, off, sink = to_dev(w)
    out = torch.empty_like(q)
    fn = lambda: attn_prefill(q, k, v, cache_off=off, window=W, sink=sink, out=out)
    r = Timer(fn, steps, warmup).run()
    flops = prefill_flops(32, 128, allowed_pairs(T, T, W))
    r.update(workload=w.name, flops_per_step=flops, value=flops / (r["ms_per_step"] * 1e-3) / 1e12,
             kernel_tflops=flops / (r["gpu_ms_per_step"] * 1e-3) / 1e12, unit="TFLOP/s")
    from oracle import attend
    rows = np.arange(T // 2, T // 2 + 1024)  # 1024 rows past the window's start, one head at a time
    pairs = float(sum(min(W, int(p) + 1) for p in rows))
    units = [lambda h=h: attend(w.q, w.k, w.v, cache_off=[0], window=W, sink=w.sink, rows=rows, heads=[h])
             for h in range(32)]
    r["cpu_baseline"] = OracleClock.run(units, [4.0 * 128 * pairs] * 32, 1e12, "TFLOP/s",
                                        "heads x 1024 rows of the window workload")
    return r


def bench_decode_and_chunk(steps, warmup, B=64):
    c = synth.decode_cache(B=B)
    k, v = c.k.to("cuda"), c.v.to("cuda")
    off = c.lengths.to("cuda")
    L = c.lengths.numpy().astype(np.int64)
    qd = c.q_decode.to("cuda")
    od = torch.empty_like(qd)
    ws = torch.empty(attn_decode_workspace_bytes(qd, k), dtype=torch.uint8, device="cuda")
    fn = lambda: attn_decode(qd, k, v, cache_off=off, workspace=ws, out=od)
    rd = Timer(fn, steps, warmup).run()
    Hkv, d, Hq = 8, 128, 32
    tk = L + 1
    kv_bytes = float((2 * Hkv * tk * d * 2).sum())
    qo_bytes = float(2 * B * Hq * d * 2)
    nbytes = kv_bytes + qo_bytes
    rd.update(workload=f"decode_bf16_B{B}_cache1024-32768_{Hq}q{Hkv}kv_d{d}", bytes_per_step=nbytes,
              value=nbytes / (rd["ms_per_step"] * 1e-3) / 1e9, kernel_GBps=nbytes / (rd["gpu_ms_per_step"] * 1e-3) / 1e9,
              unit="GB/s", mean_cache_len=float(L.mean()))
    qc = c.q_chunk.to("cuda")
    oc = torch.empty_like(qc)
    fn = lambda: attn_prefill(qc, k, v, cache_off=off, out=oc)
    rc = Timer(fn, max(3, steps // 4), max(1, warmup // 2)).run()
    pairs = float(sum(allowed_pairs(c.chunk, int(l) + c.chunk, 0) for l in L))
    flops = prefill_flops(Hq, d, pairs)
    rc.update(workload=f"chunk512_bf16_B{B}_cache1024-32768_{Hq}q{Hkv}kv_d{d}", flops_per_step=flops,
              value=flops / (rc["ms_per_step"] * 1e-3) / 1e12, kernel_tflops=flops / (rc["gpu_ms_per_step"] * 1e-3) / 1e12,
              unit="TFLOP/s")
    from oracle import attend
    sl = lambda t, b: t[b:b + 1]
    units = [lambda b=b: attend(sl(c.q_decode, b), sl(c.k, b), sl(c.v, b), cache_off=[int(L[b])]) for b in range(B)]
    work = [float(2 * Hkv * (L[b] + 1) * d * 2 + 2 * Hq * d * 2) for b in range(B)]
    rd["cpu_baseline"] = OracleClock.run(units, work, 1e9, "GB/s", "sequences (all 32 heads) of the decode step")
    units = [lambda b=b: attend(sl(c.q_chunk, b), sl(c.k, b), sl(c.v, b), cache_off=[int(L[b])], heads=[0, 11, 22])
             for b in range(B)]
    work = [prefill_flops(3, d, allowed_pairs(c.chunk, int(L[b]) + c.chunk, 0)) for b in range(B)]
    rc["cpu_baseline"] = OracleClock.run(units, work, 1e12, "TFLOP/s", "sequences x 3 heads of the 512-row chunk")
    rcs = bench_chunk_block_sparse(c, k, v, off, steps, warmup)
    del k, v
    return rd, rc, rcs


def bench_chunk_block_sparse(c, k, v, off, steps, warmup, BS=128, keep=0.05):
    """The 512-token chunk at every sequence's cache offset with query-chunked block selection
    (keep fractions 0.05 / 0.05) fused into the prefill: selection + prefill in one call."""
    B, Hq, d = c.q_chunk.shape[0], 32, 128
    qc = c.q_chunk.to("cuda")
    oc = torch.empty_like(qc)
    ws = torch.empty(attn_block_select_workspace_bytes(qc, k, BS), dtype=torch.uint8, device="cuda")
    tm = torch.empty((B, Hq), dtype=torch.float64, device="cuda")
    tr = torch.empty((B, 8), dtype=torch.float64, device="cuda")
    fn = lambda: attn_block_sparse_prefill(qc, k, v, cache_off=off, keep_mean=keep, keep_radius=keep, tau_mean=tm,
                                           tau_radius=tr, workspace=ws, out=oc)
    r = Timer(fn, max(3, steps // 2), max(1, warmup // 2)).run()
    sel = attn_block_select(qc, k, block_size=BS, cache_off=off, keep_mean=keep, keep_radius=keep)
    L = c.lengths.numpy().astype(np.int64)
    mask = sel["mask"].to(torch.int64).cpu().numpy()
    pairs = 0
    for b in range(B):  # allowed (row, key) pairs inside the kept blocks
        off_b = int(L[b])
        for qb in range(mask.shape[2]):
            r0, r1 = qb * BS, min((qb + 1) * BS, c.chunk)
            pos = np.arange(off_b + r0, off_b + r1)
            kbs = np.nonzero(mask[b, :, qb].sum(0))[0]
            for kb in kbs:
                j0, j1 = kb * BS, (kb + 1) * BS
                per_row = np.clip(np.minimum(pos + 1, j1) - j0, 0, None)
                pairs += int(mask[b, :, qb, kb].sum()) * int(per_row.sum())
    flops = 4.0 * d * pairs
    sel_bytes = float(qc.numel() * 2 + sum(8 * (int(l) + c.chunk) * d * 2 for l in L))
    r.update(workload=f"chunk512_block_sparse_bf16_B{B}_cache1024-32768_32q8kv_d128_keep{keep}", flops_per_step=flops,
             value=flops / (r["ms_per_step"] * 1e-3) / 1e12, kernel_tflops=flops / (r["gpu_ms_per_step"] * 1e-3) / 1e12,
             unit="TFLOP/s (kept pairs; selection included in the time)",
             kept_fraction=float(mask.sum()) / float(sum(Hq * sum((int(l) + min((qb + 1) * BS, c.chunk) - 1) // BS + 1
                                                             for qb in range(mask.shape[2])) for l in L)),
             select_bytes=sel_bytes)
    from oracle import attend, select_blocks
    sl = lambda t, b: t[b:b + 1]

    def unit(b):
        m = select_blocks(sl(c.q_chunk, b), sl(c.k, b), BS, cache_off=[int(L[b])], keep_mean=keep, keep_radius=keep)
        attend(sl(c.q_chunk, b), sl(c.k, b), sl(c.v, b), cache_off=[int(L[b])], heads=[0, 11, 22],
               block_mask=m["mask"], block_size=BS)

    work = [flops / B * 3 / Hq] * B  # the mean kept work of a sequence's three heads
    r["cpu_baseline"] = OracleClock.run([lambda b=b: unit(b) for b in range(B)], work, 1e12, "TFLOP/s",
                                        "sequences: selection (all heads) + 3 heads' block-sparse chunk")
    del qc
    return r


def bench_ring_decode(steps, warmup, B=64, W=1024):
    """Sliding-window decode over full W-slot ring caches (every sequence has seen more than
    W tokens), the step's K/V appended by the call."""
    Hq, Hkv, d = 32, 8, 128
    st = synth.ring_state(B, Hq, Hkv, d, W, n_lo=W, n_hi=8 * W)
    q, kn, vn = (t.to("cuda") for t in synth.ring_step(B, Hq, Hkv, d, 0))
    k_ring, v_ring, n_seen, sink = st.k.to("cuda"), st.v.to("cuda"), st.n_seen.to("cuda"), st.sink.to("cuda")
    o = torch.empty_like(q)
    ws = torch.empty(attn_ring_decode_workspace_bytes(q, k_ring), dtype=torch.uint8, device="cuda")
    fn = lambda: attn_ring_decode(q, kn, vn, k_ring, v_ring, n_seen, sink=sink, workspace=ws, out=o)
    r = Timer(fn, steps, warmup).run()
    kv_bytes = float(B * 2 * Hkv * W * d * 2)        # every filled slot's K and V row
    other = float(2 * B * Hq * d * 2 + 2 * 2 * B * Hkv * d * 2)  # q, o; new K/V read and written
    nbytes = kv_bytes + other
    r.update(workload=f"ring_decode_bf16_B{B}_W{W}_{Hq}q{Hkv}kv_d{d}", bytes_per_step=nbytes,
             value=nbytes / (r["ms_per_step"] * 1e-3) / 1e9, kernel_GBps=nbytes / (r["gpu_ms_per_step"] * 1e-3) / 1e9,
             unit="GB/s")
    from oracle.ring import RingCache, attend_unmasked
    qh, knh, vnh = (t.cpu() for t in synth.ring_step(B, Hq, Hkv, d, 0))

    def unit(b):
        rc = RingCache(Hkv, d, W)
        rc.k, rc.v, rc.n = st.k[b].double().numpy(), st.v[b].double().numpy(), int(st.n_seen[b])
        K, V = rc.add(knh[b, :, 0].double().numpy(), vnh[b, :, 0].double().numpy())
        attend_unmasked(qh[b, :, 0].double().numpy(), K, V, Hq, sink=st.sink.double().numpy())

    r["cpu_baseline"] = OracleClock.run([lambda b=b: unit(b) for b in range(B)], [nbytes / B] * B, 1e9, "GB/s",
                                        "sequences (all heads) of the ring step", budget_s=2.0)
    return r


def bench_mla_decode(steps, warmup, B=64, H=16):
    """Multi-head latent attention decode, absorbed form: batch 64, 16 heads, latent 512 +
    rope 64 per cached token, cache lengths uniform in [1024, 32768]."""
    m = synth.mla_cache(B=B, H=H)
    qn, qr, ck, kr = m.q_nope.cuda(), m.q_rope.cuda(), m.c_kv.cuda(), m.k_rope.cuda()
    wk, wv, off = m.w_uk.cuda(), m.w_uv.cuda(), m.cache_off.cuda()
    o = torch.empty((B, H, 1, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(attn_mla_decode_workspace_bytes(qn, qr, ck, kr, wv), dtype=torch.uint8, device="cuda")
    fn = lambda: attn_mla_decode(qn, qr, ck, kr, wk, wv, cache_off=off, workspace=ws, out=o)
    r = Timer(fn, steps, warmup).run()
    L = m.cache_off.numpy().astype(np.int64)
    lat_bytes = float(((L + 1) * (512 + 64) * 2).sum())  # every cached token's latent and rope key, once
    other = float(B * H * (128 + 64 + 128) * 2 + 2 * H * 512 * 128 * 2)  # q, o, w_uk, w_uv
    nbytes = lat_bytes + other
    r.update(workload=f"mla_decode_bf16_B{B}_H{H}_cache1024-32768_r512_rope64", bytes_per_step=nbytes,
             value=nbytes / (r["ms_per_step"] * 1e-3) / 1e9, kernel_GBps=nbytes / (r["gpu_ms_per_step"] * 1e-3) / 1e9,
             unit="GB/s")
    del ck, kr
    from oracle.mla import mla_absorbed
    sl = lambda t, b: t[b:b + 1]
    units = [lambda b=b: mla_absorbed(sl(m.q_nope, b), sl(m.q_rope, b), sl(m.c_kv, b), sl(m.k_rope, b), m.w_uk, m.w_uv,
                                      cache_off=sl(m.cache_off, b)) for b in range(B)]
    work = [float((L[b] + 1) * (512 + 64) * 2) for b in range(B)]
    r["cpu_baseline"] = OracleClock.run(units, work, 1e9, "GB/s", "sequences (all heads) of the MLA step", budget_s=2.0)
    return r


def bench_dsa_decode(steps, warmup, B=64, topk=2048):
    """Token top-k sparse decode: batch 64, 32 query / 8 KV heads, cache lengths uniform in
    [1024, 32768], 64 indexer heads of width 128, top 2048 tokens per query."""
    x = synth.dsa_inputs(B=B)
    q, k, v, qi, ki, wi = (t.cuda() for t in (x.q, x.k, x.v, x.qi, x.ki, x.wi))
    off, sink = x.cache_off.cuda(), x.sink.cuda()
    o = torch.empty_like(q)
    ws = torch.empty(attn_dsa_decode_workspace_bytes(q, k, topk), dtype=torch.uint8, device="cuda")
    fn = lambda: attn_dsa_decode(q, k, v, qi, ki, wi, topk, cache_off=off, sink=sink, workspace=ws, out=o)
    r = Timer(fn, steps, warmup).run()
    L = x.cache_off.numpy().astype(np.int64) + 1  # visible tokens per query
    Hkv, d, Hq, Hi = 8, 128, 32, 64
    idx_bytes = float((L * 128 * 2).sum())                                # every visible token's indexer key
    kv_bytes = float((2 * Hkv * np.minimum(L, topk) * d * 2).sum())       # the kept K and V rows
    other = float(2 * B * Hq * d * 2 + B * Hi * 128 * 2 + B * Hi * 4)    # q, o, qi, wi
    nbytes = idx_bytes + kv_bytes + other
    r.update(workload=f"dsa_decode_bf16_B{B}_cache1024-32768_{Hq}q{Hkv}kv_d{d}_idx{Hi}x128_top{topk}",
             bytes_per_step=nbytes, value=nbytes / (r["ms_per_step"] * 1e-3) / 1e9,
             kernel_GBps=nbytes / (r["gpu_ms_per_step"] * 1e-3) / 1e9, unit="GB/s")
    del k, v
    from oracle.dsa import sparse_attend
    sl = lambda t, b: t[b:b + 1]
    units = [lambda b=b: sparse_attend(sl(x.q, b), sl(x.k, b), sl(x.v, b), sl(x.qi, b), sl(x.ki, b), sl(x.wi, b), topk,
                                       cache_off=sl(x.cache_off, b), sink=x.sink) for b in range(B)]
    work = [float(L[b] * 128 * 2 + 2 * Hkv * min(L[b], topk) * d * 2) for b in range(B)]
    r["cpu_baseline"] = OracleClock.run(units, work, 1e9, "GB/s", "sequences (indexer, top-k, all heads) of the step",
                                        budget_s=2.0)
    return r


def bench_block_sparse(steps, warmup, T=65536, BS=128):
    """Block selection and block-sparse prefill at T = 65536: the selection alone, the prefill
    alone over the selection's kept lists, and the two in one call (the prefill deciding each
    key block from the selection's scores and thresholds)."""
    w = synth.block_sparse_prefill(T=T, BS=BS)
    q, k, v, _, _ = to_dev(w)
    sel_fn = lambda: attn_block_select(q, k, block_size=BS, keep_mean=w.keep_mean, keep_radius=w.keep_radius)
    rs = Timer(sel_fn, max(3, steps // 2), max(1, warmup // 2)).run()
    sel = sel_fn()
    out = torch.empty_like(q)
    fn = lambda: attn_prefill(q, k, v, block_list=sel["list"], block_size=BS, out=out)
    rp = Timer(fn, max(3, steps // 2), max(1, warmup // 2)).run()
    ws = torch.empty(attn_block_select_workspace_bytes(q, k, BS), dtype=torch.uint8, device="cuda")
    tm = torch.empty((1, 32), dtype=torch.float64, device="cuda")
    tr = torch.empty((1, 8), dtype=torch.float64, device="cuda")
    ffn = lambda: attn_block_sparse_prefill(q, k, v, keep_mean=w.keep_mean, keep_radius=w.keep_radius, tau_mean=tm,
                                            tau_radius=tr, workspace=ws, out=out)
    rf = Timer(ffn, max(3, steps // 2), max(1, warmup // 2)).run()
    m = sel["mask"].to(torch.int64)
    nb = T // BS
    diag = int(torch.diagonal(m, dim1=-2, dim2=-1).sum())
    total = int(m.sum())
    pairs = diag * block_pairs(BS, 0, 0) + (total - diag) * block_pairs(BS, 1, 0)
    flops = 4.0 * 128 * pairs
    adm = 32 * nb * (nb + 1) // 2
    sel_bytes = float(q.numel() * 2 + k.numel() * 2)
    rp.update(workload=f"block_sparse_prefill_bf16_T{T}_BS{BS}_32q8kv_d128", flops_per_step=flops,
              value=flops / (rp["ms_per_step"] * 1e-3) / 1e12, kernel_tflops=flops / (rp["gpu_ms_per_step"] * 1e-3) / 1e12,
              unit="TFLOP/s", kept_fraction=total / adm)
    rs.update(workload=f"block_select_fp64_T{T}_BS{BS}_32q8kv_d128", bytes_per_step=sel_bytes,
              value=sel_bytes / (rs["ms_per_step"] * 1e-3) / 1e9, unit="GB/s (q+k read)")
    rp["select_plus_prefill_ms"] = rs["ms_per_step"] + rp["ms_per_step"]
    rp["fused_select_prefill_ms"] = rf["ms_per_step"]
    rp["fused_select_prefill_gpu_ms"] = rf["gpu_ms_per_step"]
    from oracle import attend
    mask_h = sel["mask"].cpu().numpy()
    qbs = [64, 200, 300, 420, 511]  # query blocks (128 rows) of head 0 .. 4, one each

    def unit(i):
        h = i % 32
        rows = np.arange(qbs[i % 5] * BS, qbs[i % 5] * BS + BS)
        attend(w.q, w.k, w.v, rows=rows, heads=[h], block_mask=mask_h, block_size=BS)

    def unit_work(i):
        h, qb = i % 32, qbs[i % 5]
        kept = mask_h[0, h, qb]
        return 4.0 * 128 * (int(kept[:qb].sum()) * BS * BS + int(kept[qb]) * BS * (BS + 1) // 2)

    n = 64
    rp["cpu_baseline"] = OracleClock.run([lambda i=i: unit(i) for i in range(n)], [unit_work(i) for i in range(n)], 1e12,
                                         "TFLOP/s", "(head, 128-row query block) pieces of the block-sparse prefill")
    # the selection per KV group (its query heads and its key head, every row): thresholds are per
    # head and per KV head, so each group's selection is the workload's own
    from oracle import select_blocks
    hkv = k.shape[1]
    g = q.shape[1] // hkv

    def sel_unit(kv):
        select_blocks(w.q[:, g * kv:g * (kv + 1)], w.k[:, kv:kv + 1], BS, keep_mean=w.keep_mean,
                      keep_radius=w.keep_radius)

    rs["cpu_baseline"] = OracleClock.run([lambda kv=kv: sel_unit(kv) for kv in range(hkv)], [sel_bytes / hkv] * hkv, 1e9,
                                         "GB/s", f"KV groups ({g} query heads and their key head, all {T} rows) of the selection")
    return rs, rp


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline(w, budget_s=12.0):
    """The float64 oracle on host cores on a bounded sample of the causal-prefill workload:
    whole heads (all 8192 rows) until the time budget is spent; value in TFLOP/s of the
    same algorithmic flops."""
    from oracle import attend

    T = w.q.shape[2]
    q, k, v = w.q.double().numpy(), w.k.double().numpy(), w.v.double().numpy()
    units = [lambda h=h: attend(q, k, v, cache_off=[0], scale=w.scale, heads=[h]) for h in range(w.q.shape[1])]
    work = [4.0 * 128 * allowed_pairs(T, T, 0)] * w.q.shape[1]
    return OracleClock.run(units, work, 1e12, "TFLOP/s", f"of 32 query heads, all {T} rows each", budget_s=budget_s)


# ------------------------------------------------------------------ measured traffic
def load_traffic(path):
    """HBM bytes per launch (counter-measured, copy-calibrated) per workload, kept only for
    kernels whose source is unchanged since the counters were taken (sha256 of the file)."""
    import hashlib

    if not path or not os.path.exists(path):
        return {}
    with open(path) as f:
        data = json.load(f)
    out = {}
    for name, e in data.get("kernels", {}).items():
        src = os.path.join(ROOT, "sparse_offset_causal_amd", "csrc", e["source"])
        if not os.path.exists(src):
            continue
        with open(src, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != e["source_sha256"]:
                continue
        out[name] = e["hbm_bytes"]
    return out


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="all",
                    help="all | causal_prefill | window_sink | decode (with the chunk and its block-sparse form) | ring_decode | "
                         "mla_decode | dsa_decode | block_sparse | "
                         "copy (HBM counter calibration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="JSON file of HBM bytes per launch measured with rocprofv3 counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    torch.backends.cuda.matmul.allow_tf32 = False
    # the oracle's host timing uses every core this process may run on, BLAS threads to match
    from threadpoolctl import threadpool_limits

    OracleClock.cores = len(os.sched_getaffinity(0))
    OracleClock.enabled = not args.no_cpu_baseline
    threadpool_limits(limits=OracleClock.cores, user_api="blas")
    torch.set_num_threads(OracleClock.cores)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    if args.only == "copy":
        # A plain device-to-device copy of known size: HBM byte counters read on it give the
        # scale factor between counted and true bytes.
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        r = Timer(lambda: dst.copy_(src), args.steps, args.warmup).run()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": r["gpu_ms_per_step"],
                          "GBps_read_plus_write": 2 * n / (r["gpu_ms_per_step"] * 1e-3) / 1e9}), flush=True)
        return

    also = {}
    head = None
    w2 = None
    if args.only in ("all", "causal_prefill"):
        head, w2 = bench_causal_prefill(args.steps, args.warmup)
        log(f"causal prefill: {head['value']:.1f} TFLOP/s ({head['ms_per_step']:.3f} ms/step)")
    if args.only in ("all", "window_sink"):
        r = bench_window_sink(args.steps, args.warmup)
        also["window_sink_prefill"] = r
        log(f"window+sink prefill: {r['value']:.1f} TFLOP/s ({r['ms_per_step']:.3f} ms)")
        torch.cuda.empty_cache()
    if args.only in ("all", "decode"):
        rd, rc, rcs = bench_decode_and_chunk(args.steps, args.warmup)
        also["decode"], also["chunk_prefill"], also["chunk_block_sparse"] = rd, rc, rcs
        log(f"decode: {rd['value']:.0f} GB/s ({rd['ms_per_step']:.3f} ms); chunk: {rc['value']:.1f} TFLOP/s; "
            f"chunk block-sparse (selection included): {rcs['ms_per_step']:.3f} ms, kept {rcs['kept_fraction']:.3f}")
        torch.cuda.empty_cache()
    if args.only in ("all", "ring_decode"):
        r = bench_ring_decode(args.steps, args.warmup)
        also["ring_decode"] = r
        log(f"ring decode: {r['value']:.0f} GB/s ({r['ms_per_step']:.3f} ms)")
        torch.cuda.empty_cache()
    if args.only in ("all", "mla_decode"):
        r = bench_mla_decode(args.steps, args.warmup)
        also["mla_decode"] = r
        log(f"mla decode: {r['value']:.0f} GB/s ({r['ms_per_step']:.3f} ms)")
        torch.cuda.empty_cache()
    if args.only in ("all", "dsa_decode"):
        r = bench_dsa_decode(args.steps, args.warmup)
        also["dsa_decode"] = r
        log(f"dsa decode: {r['value']:.0f} GB/s ({r['ms_per_step']:.3f} ms)")
        torch.cuda.empty_cache()
    if args.only in ("all", "block_sparse"):
        rs, rp = bench_block_sparse(args.steps, args.warmup)
        also["block_select"], also["block_sparse_prefill"] = rs, rp
        log(f"block select: {rs['ms_per_step']:.3f} ms; block-sparse prefill {rp['value']:.1f} TFLOP/s "
            f"({rp['ms_per_step']:.3f} ms, kept {rp['kept_fraction']:.3f})")
        torch.cuda.empty_cache()

    if head is None:  # a single non-headline workload was requested: its main kernel heads the line
        for key in ("window_sink_prefill", "decode", "ring_decode", "mla_decode", "dsa_decode", "block_sparse_prefill"):
            if key in also:
                head = also[key]
                break
    roof_bound = "hbm" if head["unit"] == "GB/s" else "mfma"
    if roof_bound == "mfma":
        achieved = head["flops_per_step"] / (head["gpu_ms_per_step"] * 1e-3) / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved = head["bytes_per_step"] / (head["gpu_ms_per_step"] * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBPS, "GB/s"
    measured = load_traffic(args.traffic)
    traffic = measured.get(head["workload"])
    for r in also.values():
        if r.get("workload") in measured:
            r["hbm_bytes_per_launch_measured"] = measured[r["workload"]]
    line = {
        "metric": METRIC,
        "value": round(head["value"], 3),
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), cast to bf16; see synth/)",
        "config": {"workload": head["workload"], "batch": 1, "n_heads": 32, "n_kv": 8, "head_dim": 128,
                   "tq": 8192 if args.only in ("all", "causal_prefill") else None, "cache_offset": 0},
        "roofline": {"bound": roof_bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic},
        "also": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in r.items()} for k, r in also.items()},
    }
    if not args.no_cpu_baseline and w2 is not None:
        log("cpu baseline (float64 oracle) ...")
        line["cpu_baseline"] = cpu_baseline(w2)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
