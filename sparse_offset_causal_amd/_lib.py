"""ctypes view of libsoc_attn.so (the C ABI declared in include/soc_attn.h)."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_uint8, c_void_p

# SOC_ATTN_LIB names another build of the same library (the sanitized host build the ABI
# tests run under); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("SOC_ATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsoc_attn.so")

ATTN_BF16, ATTN_F32 = 0, 1
ATTN_OK, ATTN_E_INVAL, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_HIP = 0, -1, -2, -3, -4

EXPORTS = (
    "attn_prefill",
    "attn_decode_workspace_bytes",
    "attn_decode",
    "attn_decode_noalloc",
    "attn_decode_noalloc_max_scratch_bytes",
    "attn_ring_decode_workspace_bytes",
    "attn_ring_decode",
    "attn_mla_decode_workspace_bytes",
    "attn_mla_decode",
    "attn_dsa_decode_workspace_bytes",
    "attn_dsa_decode",
    "attn_block_select_workspace_bytes",
    "attn_block_select",
    "attn_block_list_from_mask",
    "attn_block_sparse_prefill_workspace_bytes",
    "attn_block_sparse_prefill",
    "attn_last_error",
)


class AttnStrides(ctypes.Structure):
    _fields_ = [("b", c_int64), ("h", c_int64), ("t", c_int64)]


class AttnShape(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("n_heads", c_int32), ("n_kv", c_int32), ("head_dim", c_int32),
                ("tq", c_int32), ("tk", c_int32), ("dtype", c_int)]


class AttnMlaShape(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("n_heads", c_int32), ("tq", c_int32), ("tk", c_int32),
                ("kv_rank", c_int32), ("rope_dim", c_int32), ("nope_dim", c_int32), ("v_dim", c_int32),
                ("dtype", c_int)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                           "or `python sparse_offset_causal_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    lib.attn_prefill.argtypes = [POINTER(AttnShape), P, AttnStrides, P, P, AttnStrides, P, AttnStrides,
                                 P, c_int32, P, c_float, P, P, c_int32, P]
    lib.attn_prefill.restype = c_int
    lib.attn_decode_workspace_bytes.argtypes = [POINTER(AttnShape), c_int32]
    lib.attn_decode_workspace_bytes.restype = c_size_t
    lib.attn_decode.argtypes = [POINTER(AttnShape), P, AttnStrides, P, P, AttnStrides, P, AttnStrides,
                                P, c_int32, P, c_float, P, c_size_t, c_int32, P]
    lib.attn_decode.restype = c_int
    lib.attn_decode_noalloc.argtypes = [POINTER(AttnShape), P, AttnStrides, P, P, AttnStrides, P, AttnStrides,
                                        P, c_int32, P, c_float, c_int32, P]
    lib.attn_decode_noalloc.restype = c_int
    lib.attn_decode_noalloc_max_scratch_bytes.argtypes = []
    lib.attn_decode_noalloc_max_scratch_bytes.restype = c_size_t
    lib.attn_ring_decode_workspace_bytes.argtypes = [POINTER(AttnShape), c_int32]
    lib.attn_ring_decode_workspace_bytes.restype = c_size_t
    lib.attn_ring_decode.argtypes = [POINTER(AttnShape), P, AttnStrides, P, P, AttnStrides, P, P, AttnStrides,
                                     P, AttnStrides, P, P, c_float, P, c_size_t, c_int32, P]
    lib.attn_ring_decode.restype = c_int
    lib.attn_mla_decode_workspace_bytes.argtypes = [POINTER(AttnMlaShape), c_int32]
    lib.attn_mla_decode_workspace_bytes.restype = c_size_t
    lib.attn_mla_decode.argtypes = [POINTER(AttnMlaShape), P, AttnStrides, P, AttnStrides, P, AttnStrides, P,
                                    AttnStrides, P, P, P, AttnStrides, P, c_float, P, c_size_t, c_int32, P]
    lib.attn_mla_decode.restype = c_int
    lib.attn_dsa_decode_workspace_bytes.argtypes = [POINTER(AttnShape), c_int32, c_int32]
    lib.attn_dsa_decode_workspace_bytes.restype = c_size_t
    lib.attn_dsa_decode.argtypes = [POINTER(AttnShape), P, AttnStrides, P, P, AttnStrides, P, AttnStrides, P, P,
                                    c_float, P, AttnStrides, P, AttnStrides, P, c_int32, c_int32, P, P, P, c_size_t,
                                    c_int32, P]
    lib.attn_dsa_decode.restype = c_int
    lib.attn_block_select_workspace_bytes.argtypes = [POINTER(AttnShape), c_int32]
    lib.attn_block_select_workspace_bytes.restype = c_size_t
    lib.attn_block_select.argtypes = [POINTER(AttnShape), P, AttnStrides, P, AttnStrides, P, c_int32, c_int32,
                                      c_double, c_double, P, P, P, P, P, c_size_t, P]
    lib.attn_block_select.restype = c_int
    lib.attn_block_sparse_prefill_workspace_bytes.argtypes = [POINTER(AttnShape), c_int32]
    lib.attn_block_sparse_prefill_workspace_bytes.restype = c_size_t
    lib.attn_block_sparse_prefill.argtypes = [POINTER(AttnShape), P, AttnStrides, P, P, AttnStrides, P, AttnStrides,
                                              P, c_int32, P, c_float, c_int32, c_double, c_double, P, P, P, P,
                                              c_size_t, P]
    lib.attn_block_sparse_prefill.restype = c_int
    lib.attn_block_list_from_mask.argtypes = [c_int64, c_int32, P, P, P]
    lib.attn_block_list_from_mask.restype = c_int
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load().attn_last_error().decode()


__all__ = ["AttnShape", "AttnMlaShape", "AttnStrides", "load", "last_error", "EXPORTS", "LIB_PATH", "ATTN_BF16", "ATTN_F32",
           "ATTN_OK", "ATTN_E_INVAL", "ATTN_E_UNSUPPORTED", "ATTN_E_WORKSPACE", "ATTN_E_HIP",
           "c_uint8", "c_double"]
