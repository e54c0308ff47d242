"""Binding of the benchmark's probes (libqsa_probe.so, include/qsa_probe.h).

Measurement aids, not part of the QSA path: a gather of 4 KiB blocks in the attention
stage's access pattern (the memory system's gather ceiling) and a write stream in the
score GEMM's store pattern (the ceiling of its output stream).
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._lib import PKG_DIR

PROBE_LIB_PATH = os.path.join(PKG_DIR, "libqsa_probe.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "qsa_probe.h")
SIGNATURES = {
    "qsa_probe_gather": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "qsa_probe_write": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                       ctypes.c_void_p]),
}
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build the package first")
        lib = ctypes.CDLL(PROBE_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            getattr(lib, name).restype = res
            getattr(lib, name).argtypes = args
        _lib = lib
    return _lib


def probe_gather(buf: torch.Tensor, block_ids: torch.Tensor, steps: int, sink: torch.Tensor):
    """Read the 4 KiB blocks of `buf` named by block_ids (int32 [n_waves * steps * 4] on
    the GPU), checked on the host to lie inside buf."""
    if not buf.is_contiguous() or block_ids.dtype != torch.int32 or sink.dtype != torch.int32:
        raise ValueError("contiguous buf, int32 block_ids and int32 sink expected")
    n_blocks = buf.numel() * buf.element_size() // 4096
    if block_ids.numel() % (4 * steps) or sink.numel() < 1024:
        raise ValueError("block_ids must hold n_waves * steps * 4 ids; sink >= 1024 entries")
    lo, hi = int(block_ids.min()), int(block_ids.max())
    if lo < 0 or hi >= n_blocks:
        raise ValueError(f"block ids [{lo}, {hi}] outside the {n_blocks} blocks of buf")
    n_waves = block_ids.numel() // (4 * steps)
    st = torch.cuda.current_stream(buf.device).cuda_stream
    rc = load().qsa_probe_gather(buf.data_ptr(), buf.numel() * buf.element_size(),
                                 block_ids.data_ptr(), n_waves, steps, sink.data_ptr(), st)
    if rc != 0:
        raise RuntimeError(f"qsa_probe_gather failed with status {rc}")


def probe_write(buf: torch.Tensor, nontemporal: bool = False):
    """Fill the whole of `buf` (contiguous, on the GPU, a multiple of 16 bytes)."""
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_contiguous() or nbytes % 16:
        raise ValueError("a contiguous buffer of a multiple of 16 bytes expected")
    st = torch.cuda.current_stream(buf.device).cuda_stream
    rc = load().qsa_probe_write(buf.data_ptr(), nbytes, int(bool(nontemporal)), st)
    if rc != 0:
        raise RuntimeError(f"qsa_probe_write failed with status {rc}")
