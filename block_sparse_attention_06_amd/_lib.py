"""Loads libqsa.so (built in-tree) and declares the C ABI of include/qsa.h for ctypes."""
from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libqsa.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "qsa.h")

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_F = ctypes.c_float
_Z = ctypes.c_size_t

# name -> (restype, argtypes); one entry per function declared in include/qsa.h
SIGNATURES = {
    "qsa_abi_version": (_I, []),
    "qsa_last_error": (ctypes.c_char_p, []),
    "qsa_pool_keys": (_I, [_P, _L, _L, _I, _I, _P, _L, _P]),
    "qsa_pool_keys_pe": (_I, [_P, _L, _L, _I, _I, _L, _P, _P, _L, _P]),
    "qsa_index_scores": (_I, [_I, _L, _I, _I, _I, _P, _L, _P, _L, _P, _L, _L, _L, _P, _P, _L,
                              _L, _P]),
    "qsa_topk_workspace_bytes": (_Z, [_I, _L, _L, _I, _I]),
    "qsa_topk_blocks": (_I, [_I, _L, _I, _I, _P, _L, _L, _L, _L, _P, _P, _P, _Z, _P]),
    "qsa_sparse_attn_fwd": (_I, [_L, _L, _I, _I, _I, _I, _I, _P, _P, _P, _P, _L, _F, _P, _P,
                                 _P]),
    "qsa_sparse_attn_fwd_tiled": (_I, [_L, _L, _I, _I, _I, _I, _I, _P, _P, _P, _P, _L, _F, _I,
                                       _P, _P, _P]),
    "qsa_sparse_attn_fwd_rows_per_launch": (_L, [_I, _I]),
    "qsa_sparse_attn_bwd_workspace_bytes": (_Z, [_L, _L, _I, _I, _I]),
    "qsa_sparse_attn_bwd": (_I, [_L, _L, _I, _I, _I, _I, _I, _P, _P, _P, _P, _L, _F, _P, _P, _P,
                                 _P, _P, _P, _P, _Z, _P]),
    "qsa_indexer_kl_target": (_I, [_L, _L, _I, _I, _I, _I, _P, _P, _L, _F, _P, _P, _L, _P]),
    "qsa_indexer_kl_loss": (_I, [_L, _L, _I, _L, _P, _P, _L, _P, _P, _P]),
    "qsa_index_scores_bwd": (_I, [_L, _I, _I, _I, _P, _P, _P, _L, _L, _P, _L, _P, _P, _P, _P,
                                  _L, _P]),
    "qsa_sparse_attn_decode_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "qsa_sparse_attn_decode": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _L, _L, _P, _P, _F, _P,
                                    _P, _P, _Z, _P]),
    "qsa_prefill_workspace_bytes": (_Z, [_L, _L, _I, _I, _L]),
    "qsa_prefill_select": (_I, [_L, _L, _L, _I, _I, _I, _I, _P, _P, _P, _L, _P, _P, _P, _L, _P,
                                _Z, _P, _P]),
    "qsa_prefill_fused_workspace_bytes": (_Z, [_L, _L, _I, _I, _L]),
    "qsa_prefill_select_fused": (_I, [_L, _L, _L, _I, _I, _I, _I, _P, _P, _P, _L, _P, _P, _P,
                                      _L, _P, _Z, _P, _P, _P]),
    "qsa_prefill_forward": (_I, [_L, _L, _L, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                                 _L, _P, _P, _F, _P, _P, _P, _L, _P, _Z, _P, _P]),
    "qsa_prefill_varlen_workspace_bytes": (_Z, [_I, _L, _L, _I, _I, _L]),
    "qsa_prefill_varlen_select": (_I, [_I, _P, _P, _L, _L, _I, _I, _I, _I, _P, _P, _P, _P, _P,
                                       _L, _P, _Z, _P, _P]),
    "qsa_sparse_attn_varlen_fwd": (_I, [_I, _P, _P, _L, _L, _I, _I, _I, _I, _I, _P, _P, _P, _P,
                                        _F, _P, _P, _P]),
    "qsa_sparse_attn_fwd_launches": (_L, [_L, _L, _I, _I]),
    "qsa_prefill_varlen_forward": (_I, [_I, _P, _P, _L, _L, _L, _I, _I, _I, _I, _I, _I, _I, _P,
                                        _P, _P, _P, _P, _P, _P, _F, _P, _P, _P, _L, _P, _Z, _P,
                                        _P]),
    "qsa_sparse_attn_decode_paged": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _L, _I, _P, _L,
                                          _L, _P, _P, _F, _P, _P, _P, _Z, _P]),
    "qsa_decode_forward_paged": (_I, [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _L, _P,
                                      _P, _L, _I, _P, _L, _L, _P, _F, _P, _P, _P, _P, _Z, _P]),
    "qsa_decode_workspace_bytes": (_Z, [_I, _I, _I, _L, _I, _I]),
    "qsa_decode_forward_noalloc": (_I, [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _L, _P,
                                        _P, _L, _L, _P, _F, _P, _P, _P, _P]),
    "qsa_decode_forward": (_I, [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _L, _P, _P, _L,
                                _L, _P, _F, _P, _P, _P, _P, _Z, _P]),
}

_lib = None


def header_functions(path: str = HEADER_PATH) -> list:
    """Names of the functions declared in the public header."""
    with open(path) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z0-9_]+)\s*\(", text)))


def load() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
            "g.build()'` (hipcc, gfx950). The QSA path has no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
