"""Float64 CPU oracle for offset-causal attention and block selection.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constant tables) and never imports the
``sparse_offset_causal_amd`` package.

Modules
-------
attend  the plain definition of masked scaled-dot-product attention with
        absolute-position causality, window, grouped-query sharing, sink and an
        optional block mask (row-blocked through BLAS, exact per row).
select  block selection by a mean-centroid score OR'd with a max-key-radius
        score, each with its own per-head order-statistic threshold, taken step
        by step.
ring    a W-slot ring-buffer KV cache, an independent route to the window rule.
mla     multi-head latent attention, plain (keys and values rebuilt per head) and
        absorbed (query moved into latent space, one shared latent KV head).
dsa     token top-k sparse attention: an indexer's scores, the kept set per query
        token, attention over it.
brute   pure-Python scalar loops for tiny shapes (a second, independent
        implementation of both definitions).

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants the pages state, a library routine, the pages' printed mask figure,
and brute force.  Parity status of each function is listed there; no function
here is "parity unpinned".
"""
from .attend import attend, key_allowed, allowed_pair_count  # noqa: F401
from .select import select_blocks, block_list_from_mask  # noqa: F401
