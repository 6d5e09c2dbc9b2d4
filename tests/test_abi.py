"""C-ABI checks that need no GPU: the library loads, exports every function the header
declares, and rejects bad arguments with the documented codes before queueing work."""
import ctypes
import os
import re

import pytest

from sparse_offset_causal_amd import _lib
from sparse_offset_causal_amd._lib import (ATTN_BF16, ATTN_E_INVAL, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_F32,
                                           AttnShape, AttnStrides)

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "soc_attn.h")
FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation or is a no-op


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(attn_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_exported_symbols_via_nm():
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def S(b=1, h=8, kv=2, d=128, tq=16, tk=64, dt=ATTN_BF16):
    return AttnShape(b, h, kv, d, tq, tk, dt)


def st(d=128, t=None, tk=64, h=8):
    t = d if t is None else t
    return AttnStrides(h * tk * d, tk * d, t)


def prefill(lib, shape, q=FAKE, k=FAKE, v=FAKE, o=FAKE, qs=None, kvs=None, os_=None, window=0, block_list=None,
            block_size=128, block_mask=None):
    qs = qs or st()
    kvs = kvs or st()
    os_ = os_ or st()
    return lib.attn_prefill(ctypes.byref(shape), q, qs, k, v, kvs, o, os_, None, window, None, 0.0, block_mask,
                            block_list, block_size, None)


def test_invalid_shapes(lib):
    assert lib.attn_prefill(None, FAKE, st(), FAKE, FAKE, st(), FAKE, st(), None, 0, None, 0.0, None, None, 0,
                            None) == ATTN_E_INVAL
    assert prefill(lib, S(h=6, kv=4)) == ATTN_E_INVAL
    assert "multiple of n_kv" in _lib.last_error()
    assert prefill(lib, S(tq=65, tk=64)) == ATTN_E_INVAL
    assert "tq > tk" in _lib.last_error()
    assert prefill(lib, S(b=-1)) == ATTN_E_INVAL
    assert prefill(lib, S(kv=0)) == ATTN_E_INVAL


def test_unsupported_combinations(lib):
    assert prefill(lib, S(d=64)) == ATTN_E_UNSUPPORTED
    assert prefill(lib, S(d=48, dt=ATTN_F32)) == ATTN_E_UNSUPPORTED
    assert prefill(lib, S(), block_list=FAKE, block_size=64) == ATTN_E_UNSUPPORTED
    assert prefill(lib, S(), block_list=FAKE, block_size=0) == ATTN_E_INVAL
    assert prefill(lib, S(), block_mask=FAKE, block_size=64) == ATTN_E_UNSUPPORTED
    assert prefill(lib, S(), block_mask=FAKE, block_list=FAKE) == ATTN_E_INVAL
    assert "not both" in _lib.last_error()
    shape = AttnShape(1, 32, 4, 128, 8, 64, ATTN_BF16)  # 8 query heads per KV head x 8 rows = 64 > 32
    ws = lib.attn_decode_workspace_bytes(ctypes.byref(shape), 0)
    rc = lib.attn_decode(ctypes.byref(shape), FAKE, st(h=32), FAKE, FAKE, st(h=4), FAKE, st(h=32), None, 0, None,
                         0.0, FAKE, ws, 0, None)
    assert rc == ATTN_E_UNSUPPORTED


def test_null_and_misaligned_pointers(lib):
    assert prefill(lib, S(), q=None) == ATTN_E_INVAL
    assert prefill(lib, S(), o=None) == ATTN_E_INVAL
    assert prefill(lib, S(), k=FAKE + 2) == ATTN_E_INVAL
    assert "16-byte" in _lib.last_error()
    assert prefill(lib, S(), qs=AttnStrides(8192, 1024, 130)) == ATTN_E_INVAL


def test_bf16_zero_token_stride_is_rejected(lib):
    # the bf16 kernels address K/V through buffer ranges of rows x token stride bytes: a zero
    # stride (one row broadcast over the tokens) would read zeros, so it is refused
    assert prefill(lib, S(), kvs=AttnStrides(2 * 64 * 128, 64 * 128, 0)) == ATTN_E_UNSUPPORTED
    assert "token stride" in _lib.last_error()
    shape = S(tq=1, tk=1024)
    need = lib.attn_ring_decode_workspace_bytes(ctypes.byref(shape), 256)
    rc = lib.attn_ring_decode(ctypes.byref(shape), FAKE, st(tk=1), FAKE, FAKE, st(tk=1, h=2), FAKE, FAKE,
                              AttnStrides(2 * 1024 * 128, 1024 * 128, 0), FAKE, st(tk=1), FAKE, None, 0.0, FAKE, need,
                              256, None)
    assert rc == ATTN_E_UNSUPPORTED


def test_zero_sized_calls_are_noops(lib):
    assert prefill(lib, S(tq=0)) == 0
    assert prefill(lib, S(b=0), q=None, k=None, v=None, o=None) == 0
    assert _lib.last_error() == ""


def test_decode_workspace_checks(lib):
    shape = S(tq=1, tk=5000)
    need = lib.attn_decode_workspace_bytes(ctypes.byref(shape), 1024)
    assert need == ((1 * 8 * 1 * 5 * (128 + 2) * 4 + 255) // 256) * 256
    assert lib.attn_decode_workspace_bytes(ctypes.byref(S(h=6, kv=4)), 0) == 0
    args = (ctypes.byref(shape), FAKE, st(tk=5000), FAKE, FAKE, st(tk=5000), FAKE, st(tk=5000), None, 0, None, 0.0)
    assert lib.attn_decode(*args, None, need, 1024, None) == ATTN_E_WORKSPACE
    assert lib.attn_decode(*args, FAKE, need - 1, 1024, None) == ATTN_E_WORKSPACE
    assert "too small" in _lib.last_error()


def test_ring_decode_checks(lib):
    shape = S(tq=1, tk=1024)
    need = lib.attn_ring_decode_workspace_bytes(ctypes.byref(shape), 256)
    assert need == lib.attn_decode_workspace_bytes(ctypes.byref(shape), 256) + 256
    assert lib.attn_ring_decode_workspace_bytes(ctypes.byref(S(h=6, kv=4)), 0) == 0

    def call(**kw):
        sh = kw.get("shape", shape)
        return lib.attn_ring_decode(ctypes.byref(sh), FAKE, st(tk=1), kw.get("kn", FAKE), FAKE, st(tk=1, h=2),
                                    FAKE, FAKE, st(tk=1024, h=2), FAKE, st(tk=1), kw.get("ns", FAKE), None, 0.0,
                                    kw.get("ws", FAKE), kw.get("wsb", need), 256, None)

    assert call(shape=S(tq=2, tk=1024)) == ATTN_E_INVAL
    assert "tq = 1" in _lib.last_error()
    assert call(kn=None) == ATTN_E_INVAL
    assert call(ns=None) == ATTN_E_INVAL
    assert call(kn=FAKE + 4) == ATTN_E_INVAL
    assert call(ws=None) == ATTN_E_WORKSPACE
    assert call(wsb=need - 1) == ATTN_E_WORKSPACE
    assert call(shape=S(d=64, tq=1, tk=1024)) == ATTN_E_UNSUPPORTED
    assert call(shape=S(b=0, tq=1, tk=1024), kn=None, ns=None, ws=None) == 0


def test_block_select_checks(lib):
    shape = S(tq=256, tk=256)
    need = lib.attn_block_select_workspace_bytes(ctypes.byref(shape), 128)
    assert need > 0
    call = lambda **kw: lib.attn_block_select(
        ctypes.byref(kw.get("shape", shape)), FAKE, st(tk=256), FAKE, st(tk=256), None, 0, kw.get("bs", 128),
        kw.get("km", 0.05), kw.get("kr", 0.05), kw.get("tm", FAKE), FAKE, kw.get("mask", FAKE), None,
        kw.get("ws", FAKE), kw.get("wsb", need), None)
    assert call(bs=0) == ATTN_E_INVAL
    assert call(mask=None) == ATTN_E_INVAL
    assert call(tm=None) == ATTN_E_INVAL
    assert call(wsb=need - 8) == ATTN_E_WORKSPACE
    assert call(ws=None) == ATTN_E_WORKSPACE
    assert call(km=float("nan")) == ATTN_E_INVAL
    assert call(shape=S(d=32, tq=256, tk=256)) == ATTN_E_UNSUPPORTED
    assert lib.attn_block_list_from_mask(4, 0, FAKE, FAKE, None) == ATTN_E_INVAL
    assert lib.attn_block_list_from_mask(0, 4, None, None, None) == 0


def test_python_binding_rejects_cpu_tensors():
    import torch

    import sparse_offset_causal_amd as soc

    q = torch.zeros(1, 8, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        soc.attn_prefill(q, q[:, :2], q[:, :2])
