"""Python binding of libqsa: argument marshalling only.

Each function has the name of the C entry point it calls (include/qsa.h), takes torch
tensors already on the GPU, allocates outputs and workspaces with torch, and enqueues
the call on torch's current stream. Every step of the computation runs in the HIP
library; nothing here computes, and there is no fallback when the library is absent.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib

QSA_OK = 0


class QSAError(RuntimeError):
    """A libqsa entry point returned a non-OK status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def _call(name: str, *args) -> None:
    lib = _lib.load()
    st = getattr(lib, name)(*args)
    if st != QSA_OK:
        raise QSAError(name, st, lib.qsa_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (the QSA path has no CPU implementation)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def score_ld(nblk: int) -> int:
    return (nblk + 3) // 4 * 4


# Selection chunk when the caller gives none: as many rows as keep the chunk's fp32
# score rows within 8 GiB, from 4096 up to 65536. At 128K (32768 blocks) that is 65536
# rows, where a prefill step on MI355X takes 42.9 ms against 43.4 at 16384 and 44.1 at
# 8192 (fewer launches; for the fused selection, more workgroups than the GPU holds,
# so the long row tiles' CUs are refilled); at 1M it is 8192.
SCORE_CHUNK_BYTES = 8 << 30


def default_row_chunk(lq: int, lk: int, r: int = 4) -> int:
    """Rows per selection chunk for lq query rows over lk keys (see SCORE_CHUNK_BYTES)."""
    per_row = score_ld(lk // r) * 4
    rc = max(4096, min(65536, SCORE_CHUNK_BYTES // max(per_row, 1)))
    return int(max(1, min(rc, lq)))


def abi_version() -> int:
    return _lib.load().qsa_abi_version()


# ------------------------------------------------------------------------------------
# Stages
# ------------------------------------------------------------------------------------


class _PooledPe(ctypes.Structure):
    _fields_ = [("rope_dim", ctypes.c_int), ("rope_theta", ctypes.c_float)]


def _pe_arg(pe):
    """(rope_dim, rope_theta) or None -> a pointer to the C struct (kept alive by the
    returned holder) or NULL."""
    if pe is None:
        return None, None
    st = _PooledPe(int(pe[0]), float(pe[1]))
    return st, ctypes.cast(ctypes.pointer(st), ctypes.c_void_p)


def qsa_pool_keys(k_idx: torch.Tensor, r: int = 4, out: Optional[torch.Tensor] = None, *,
                  pe=None, first_block: int = 0):
    """Mean-pool [n_tok, d_I] bf16 indexer keys into [n_tok // r, d_I] (complete blocks).
    pe = (rope_dim, rope_theta) also encodes each block at position
    (first_block + b) * r (see include/qsa.h)."""
    _need(k_idx, "k_idx", torch.bfloat16, contiguous=False)
    if k_idx.dim() != 2 or k_idx.stride(1) != 1:
        raise ValueError("k_idx must be [n_tokens, d_idx] with unit column stride")
    nb, d_i = k_idx.shape[0] // r, k_idx.shape[1]
    if out is None:
        out = torch.empty((nb, d_i), dtype=torch.bfloat16, device=k_idx.device)
    _need(out, "out", torch.bfloat16, k_idx.device, contiguous=False)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] < nb or out.shape[1] != d_i:
        raise ValueError("out must be [>= n_tokens // r, d_idx] with unit column stride")
    if pe is None:
        _call("qsa_pool_keys", _ptr(k_idx), k_idx.stride(0), nb, d_i, r, _ptr(out),
              out.stride(0), _stream(k_idx))
    else:
        keep, pp = _pe_arg(pe)
        _call("qsa_pool_keys_pe", _ptr(k_idx), k_idx.stride(0), nb, d_i, r, first_block, pp,
              _ptr(out), out.stride(0), _stream(k_idx))
        del keep
    return out


def qsa_index_scores(q_idx: torch.Tensor, w: torch.Tensor, k_pooled: torch.Tensor, *,
                     q_pos0: int = 0, seq_lens: Optional[torch.Tensor] = None, r: int = 4,
                     nblk: Optional[int] = None, out: Optional[torch.Tensor] = None):
    """Block scores. Unbatched: q_idx [Lq,H,dI], w [Lq,H], k_pooled [nblk,dI] -> [Lq, ld].
    Batched: q_idx [B,Lq,H,dI], w [B,Lq,H], k_pooled [B,nblk,dI] -> [B, Lq, ld]."""
    batched = q_idx.dim() == 4
    qb = q_idx if batched else q_idx.unsqueeze(0)
    wb = w if batched else w.unsqueeze(0)
    kb = k_pooled if batched else k_pooled.unsqueeze(0)
    _need(qb, "q_idx", torch.bfloat16)
    _need(wb, "w", torch.float32, qb.device)
    _need(kb, "k_pooled", torch.bfloat16, qb.device)
    bsz, lq, h, di = qb.shape
    nblk = kb.shape[1] if nblk is None else nblk
    if nblk > kb.shape[1] or kb.shape[0] != bsz or wb.shape != (bsz, lq, h):
        raise ValueError("inconsistent shapes")
    ld = score_ld(nblk)
    if out is None:
        out = torch.empty((bsz, lq, ld), dtype=torch.float32, device=qb.device)
    ob = out if out.dim() == 3 else out.unsqueeze(0)
    _need(ob, "out", torch.float32, qb.device)
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32, qb.device)
    _call("qsa_index_scores", bsz, lq, h, di, r, _ptr(qb), qb.stride(0), _ptr(wb), wb.stride(0),
          _ptr(kb), kb.stride(0), nblk, q_pos0, _ptr(seq_lens), _ptr(ob), ob.shape[2],
          ob.stride(0), _stream(qb))
    return out if batched or out.dim() == 2 else out[0]


def qsa_topk_blocks(scores: torch.Tensor, *, lq: int, nblk: int, budget: int, q_pos0: int = 0,
                    seq_lens: Optional[torch.Tensor] = None, r: int = 4,
                    out: Optional[torch.Tensor] = None):
    """Kept block ids per query row: scores [Lq, ld] or [B, Lq, ld] -> int32 [(B,) Lq, budget/r]."""
    batched = scores.dim() == 3
    sb = scores if batched else scores.unsqueeze(0)
    _need(sb, "scores", torch.float32)
    bsz = sb.shape[0]
    n_sel = budget // r
    if out is None:
        out = torch.empty((bsz, lq, n_sel), dtype=torch.int32, device=sb.device)
    _need(out, "out", torch.int32, sb.device)
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32, sb.device)
    ws_bytes = _lib.load().qsa_topk_workspace_bytes(bsz, lq, nblk, budget, r)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=sb.device) if ws_bytes else None
    _call("qsa_topk_blocks", bsz, lq, r, budget, _ptr(sb), sb.shape[2], sb.stride(0), nblk,
          q_pos0, _ptr(seq_lens), _ptr(out), _ptr(ws), ws_bytes, _stream(sb))
    return out if batched else out.view(lq, n_sel)


def qsa_sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sel: torch.Tensor, *,
                        q_pos0: int = 0, scale: Optional[float] = None, r: int = 4,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        want_lse: bool = True):
    """Prefill attention over the kept tokens. q [Lq,Hq,d], k/v [Lk,Hkv,d], sel [Lq,n_sel]."""
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, q.device)
    _need(v, "v", torch.bfloat16, q.device)
    _need(sel, "sel", torch.int32, q.device)
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((lq, hq), dtype=torch.float32, device=q.device)
    _call("qsa_sparse_attn_fwd", lq, lk, hq, hkv, d, r, sel.shape[1], _ptr(q), _ptr(k), _ptr(v),
          _ptr(sel), q_pos0, scale, _ptr(out), _ptr(lse), _stream(q))
    return out, lse


def qsa_sparse_attn_fwd_tiled(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                              sel: torch.Tensor, *, q_pos0: int = 0, scale: Optional[float] = None,
                              r: int = 4, min_shared: int = 0, out: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None, want_lse: bool = True):
    """qsa_sparse_attn_fwd as four-row tiles that stage the union of their kept blocks
    in LDS (min_shared: 0 always, 1..64 when that many of 64 sampled blocks are shared,
    65 never). n_sel <= 512."""
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, q.device)
    _need(v, "v", torch.bfloat16, q.device)
    _need(sel, "sel", torch.int32, q.device)
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((lq, hq), dtype=torch.float32, device=q.device)
    _call("qsa_sparse_attn_fwd_tiled", lq, lk, hq, hkv, d, r, sel.shape[1], _ptr(q), _ptr(k),
          _ptr(v), _ptr(sel), q_pos0, scale, min_shared, _ptr(out), _ptr(lse), _stream(q))
    return out, lse


def qsa_sparse_attn_fwd_rows_per_launch(hkv: int, d: int, device=None) -> int:
    """Rows per GPU launch of qsa_sparse_attn_fwd on `device` (the current device by
    default); -1 when the runtime cannot report the occupancy, 0 for unsupported
    arguments."""
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        return int(_lib.load().qsa_sparse_attn_fwd_rows_per_launch(hkv, d))


def qsa_sparse_attn_fwd_launches(lq: int, lk: int, hkv: int, d: int, device=None) -> int:
    """Kernel launches one qsa_sparse_attn_fwd call issues for lq rows over lk keys on
    `device` (the current device by default)."""
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        return int(_lib.load().qsa_sparse_attn_fwd_launches(lq, lk, hkv, d))


def qsa_sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sel: torch.Tensor,
                        out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor, *,
                        q_pos0: int = 0, scale: Optional[float] = None, r: int = 4,
                        workspace: Optional[torch.Tensor] = None):
    """Gradients of qsa_sparse_attn_fwd with respect to q, k, v over the same selection.

    out/lse are the forward's outputs, dout [Lq,Hq,d] bf16 the output gradient.
    Returns fp32 (dq [Lq,Hq,d], dk [Lk,Hkv,d], dv [Lk,Hkv,d])."""
    _need(q, "q", torch.bfloat16)
    for name, t, dt in (("k", k, torch.bfloat16), ("v", v, torch.bfloat16), ("sel", sel, torch.int32),
                        ("out", out, torch.bfloat16), ("lse", lse, torch.float32),
                        ("dout", dout, torch.bfloat16)):
        _need(t, name, dt, q.device)
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    n_sel = sel.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = torch.empty((lq, hq, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((lk, hkv, d), dtype=torch.float32, device=q.device)
    dv = torch.empty((lk, hkv, d), dtype=torch.float32, device=q.device)
    nbytes = _lib.load().qsa_sparse_attn_bwd_workspace_bytes(lq, lk, hq, r, n_sel)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _call("qsa_sparse_attn_bwd", lq, lk, hq, hkv, d, r, n_sel, _ptr(q), _ptr(k), _ptr(v),
          _ptr(sel), q_pos0, scale, _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
          _ptr(dv), _ptr(workspace), workspace.numel(), _stream(q))
    return dq, dk, dv


def qsa_indexer_kl_target(q: torch.Tensor, k: torch.Tensor, *, q_pos0: int = 0,
                          scale: Optional[float] = None, r: int = 4):
    """Dense attention statistics for the indexer warm-up: (lse [Lq,Hq], target [Lq, ld])
    with target the unnormalised block max of the head-summed probabilities."""
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, q.device)
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    ld = score_ld(lk // r)
    lse = torch.empty((lq, hq), dtype=torch.float32, device=q.device)
    target = torch.empty((lq, ld), dtype=torch.float32, device=q.device)
    _call("qsa_indexer_kl_target", lq, lk, hq, hkv, d, r, _ptr(q), _ptr(k), q_pos0, scale,
          _ptr(lse), _ptr(target), ld, _stream(q))
    return lse, target


def qsa_indexer_kl_loss(scores: torch.Tensor, target: torch.Tensor, *, nblk: int,
                        q_pos0: int = 0, r: int = 4):
    """KL(target || softmax(scores)) per row over its scored blocks, and dL/dscores."""
    _need(scores, "scores", torch.float32)
    _need(target, "target", torch.float32, scores.device)
    lq, ld = scores.shape
    if target.shape != scores.shape:
        raise ValueError("scores and target must have the same shape")
    loss = torch.empty(lq, dtype=torch.float32, device=scores.device)
    dscores = torch.empty_like(scores)
    _call("qsa_indexer_kl_loss", lq, nblk, r, q_pos0, _ptr(scores), _ptr(target), ld,
          _ptr(loss), _ptr(dscores), _stream(scores))
    return loss, dscores


def qsa_index_scores_bwd(q_idx: torch.Tensor, w: torch.Tensor, k_pooled: torch.Tensor,
                         dscores: torch.Tensor, *, q_pos0: int = 0, r: int = 4,
                         nblk: Optional[int] = None, n_tokens: Optional[int] = None):
    """Gradients of the block scores: (dq_idx, dw, dk_pooled[, dk_idx]) in fp32.
    q_idx [Lq,H,dI], w [Lq,H], k_pooled [nblk,dI], dscores [Lq, ld]. With n_tokens, also
    the raw indexer keys' gradient [n_tokens, dI] through the mean pooling."""
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(w, "w", torch.float32, q_idx.device)
    _need(k_pooled, "k_pooled", torch.bfloat16, q_idx.device)
    _need(dscores, "dscores", torch.float32, q_idx.device)
    lq, h, di = q_idx.shape
    nblk = k_pooled.shape[0] if nblk is None else nblk
    dq = torch.empty((lq, h, di), dtype=torch.float32, device=q_idx.device)
    dw = torch.empty((lq, h), dtype=torch.float32, device=q_idx.device)
    dkp = torch.empty((max(nblk, 1), di), dtype=torch.float32, device=q_idx.device)
    dki = None if n_tokens is None else torch.empty((n_tokens, di), dtype=torch.float32,
                                                    device=q_idx.device)
    _call("qsa_index_scores_bwd", lq, h, di, r, _ptr(q_idx), _ptr(w), _ptr(k_pooled), nblk,
          q_pos0, _ptr(dscores), dscores.shape[1], _ptr(dq), _ptr(dw), _ptr(dkp), _ptr(dki),
          0 if n_tokens is None else n_tokens, _stream(q_idx))
    return (dq, dw, dkp[:nblk]) if dki is None else (dq, dw, dkp[:nblk], dki)


def qsa_sparse_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           seq_lens: torch.Tensor, sel: torch.Tensor, *,
                           scale: Optional[float] = None, r: int = 4):
    """Decode attention: q [B,Hq,d], caches [B,Lmax,Hkv,d], seq_lens [B], sel [B,n_sel]."""
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, q.device)
    _need(v_cache, "v_cache", torch.bfloat16, q.device)
    _need(seq_lens, "seq_lens", torch.int32, q.device)
    _need(sel, "sel", torch.int32, q.device)
    bsz, hq, d = q.shape
    _, lmax, hkv, _ = k_cache.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    n_sel = sel.shape[-1]
    out = torch.empty_like(q)
    lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    ws_bytes = _lib.load().qsa_sparse_attn_decode_workspace_bytes(bsz, hq, d, n_sel)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _call("qsa_sparse_attn_decode", bsz, hq, hkv, d, r, n_sel, _ptr(q), _ptr(k_cache),
          _ptr(v_cache), k_cache.stride(0), lmax, _ptr(seq_lens), _ptr(sel), scale, _ptr(out),
          _ptr(lse), _ptr(ws), ws_bytes, _stream(q))
    return out, lse


# ------------------------------------------------------------------------------------
# Whole paths
# ------------------------------------------------------------------------------------


# Sequences with more blocks than this take the fused selection by default: there it
# is faster (measured on MI355X, per 128K prefill step: 4.2 against 4.5 ms of
# selection in 65536-row chunks, 4.7 against 5.1 ms in 16384-row chunks; 8192 rows
# over 1M keys: 2.8 against 4.2 ms), while shorter ones are selected faster by the
# two-kernel path (32K: 9.73 against 9.50 ms a whole step).
FUSED_MIN_BLOCKS = 16384


def prefer_fused_select(lk: int, r: int = 4) -> bool:
    """The default selection path for a prefill over lk keys."""
    return lk // r > FUSED_MIN_BLOCKS


class PrefillPlan:
    """Preallocated outputs and workspace for repeated prefill calls of one shape.
    fused: the selection path the plan is sized for (None: prefer_fused_select)."""

    def __init__(self, lq, lk, hq, hkv, d, h_idx, d_idx, budget, *, r=4, row_chunk=None,
                 device="cuda", with_attention=True, fused=None):
        self.shape = (lq, lk, hq, hkv, d, h_idx, d_idx, budget, r)
        row_chunk = default_row_chunk(lq, lk, r) if row_chunk is None else row_chunk
        self.row_chunk = row_chunk
        fused = prefer_fused_select(lk, r) if fused is None else fused
        self.fused = fused
        dev = torch.device(device)
        self.sel = torch.empty((lq, budget // r), dtype=torch.int32, device=dev)
        self.out = self.lse = None
        if with_attention:
            self.out = torch.empty((lq, hq, d), dtype=torch.bfloat16, device=dev)
            self.lse = torch.empty((lq, hq), dtype=torch.float32, device=dev)
        self.k_pooled = torch.empty((lk // r, d_idx), dtype=torch.bfloat16, device=dev)
        lib = _lib.load()
        nbytes = (lib.qsa_prefill_fused_workspace_bytes if fused
                  else lib.qsa_prefill_workspace_bytes)(lq, lk, r, budget, row_chunk)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        self.ws_bytes = nbytes


def _prefill_args(q_idx, w, k_idx, k_pooled_prefix, r, lk):
    for name, t, dt in (("q_idx", q_idx, torch.bfloat16), ("w", w, torch.float32),
                        ("k_idx", k_idx, torch.bfloat16)):
        _need(t, name, dt, q_idx.device)
    prefix_blocks = 0 if k_pooled_prefix is None else k_pooled_prefix.shape[0]
    if k_pooled_prefix is not None:
        _need(k_pooled_prefix, "k_pooled_prefix", torch.bfloat16, q_idx.device)
    if k_idx.shape[0] != lk - prefix_blocks * r:
        raise ValueError("k_idx must hold the indexer keys of every token after the prefix")
    return prefix_blocks


class _FusedTuning(ctypes.Structure):
    _fields_ = [("target", ctypes.c_int), ("sample_k", ctypes.c_int), ("cap", ctypes.c_int)]


def qsa_prefill_select(q_idx, w, k_idx, *, lk: int, budget: int, q_pos0: int = 0,
                       k_pooled_prefix: Optional[torch.Tensor] = None, r: int = 4,
                       row_chunk: Optional[int] = None, plan: Optional[PrefillPlan] = None,
                       pe=None, fused: Optional[bool] = None, tuning=None):
    """Selection half of prefill: pool the new blocks, score + top-k in row chunks
    (row_chunk rows each; default_row_chunk when not given, the plan's when a plan is).
    fused (default: the plan's choice, else prefer_fused_select) takes the fused
    score/top-k path, whose selection is identical; tuning = (target, sample_k, cap)
    adjusts it (0 keeps a default). Returns (sel, k_pooled)."""
    lq, h_idx, d_idx = q_idx.shape
    prefix_blocks = _prefill_args(q_idx, w, k_idx, k_pooled_prefix, r, lk)
    if fused is None:
        fused = plan.fused if plan is not None else prefer_fused_select(lk, r)
    if plan is None:
        plan = PrefillPlan(lq, lk, 1, 1, 128, h_idx, d_idx, budget, r=r, row_chunk=row_chunk,
                           device=q_idx.device, with_attention=False, fused=fused)
    if fused and not plan.fused:
        raise ValueError("the plan's workspace is not sized for the fused selection")
    keep, pp = _pe_arg(pe)
    if fused:
        tn = None if tuning is None else _FusedTuning(*[int(x) for x in tuning])
        tp = None if tn is None else ctypes.cast(ctypes.pointer(tn), ctypes.c_void_p)
        _call("qsa_prefill_select_fused", lq, lk, q_pos0, h_idx, d_idx, r, budget, _ptr(q_idx),
              _ptr(w), _ptr(k_idx), prefix_blocks * r, _ptr(k_pooled_prefix),
              _ptr(plan.k_pooled), _ptr(plan.sel), plan.row_chunk, _ptr(plan.ws), plan.ws_bytes,
              pp, tp, _stream(q_idx))
        del tn
    else:
        _call("qsa_prefill_select", lq, lk, q_pos0, h_idx, d_idx, r, budget, _ptr(q_idx),
              _ptr(w), _ptr(k_idx), prefix_blocks * r, _ptr(k_pooled_prefix),
              _ptr(plan.k_pooled), _ptr(plan.sel), plan.row_chunk, _ptr(plan.ws), plan.ws_bytes,
              pp, _stream(q_idx))
    del keep
    return plan.sel, plan.k_pooled


def qsa_prefill_forward(q, k, v, q_idx, w, k_idx, *, budget: int, q_pos0: int = 0,
                        k_pooled_prefix: Optional[torch.Tensor] = None,
                        scale: Optional[float] = None, r: int = 4,
                        row_chunk: Optional[int] = None, plan: Optional[PrefillPlan] = None,
                        pe=None):
    """Whole prefill: pool the new blocks, score + top-k in row chunks, attention.

    q [Lq,Hq,d], k/v [Lk,Hkv,d], q_idx [Lq,H_I,d_I], w [Lq,H_I]; k_idx holds the raw
    indexer keys of tokens P*r .. Lk-1 where P = rows of k_pooled_prefix (or 0).
    Returns (out, lse, sel, k_pooled).
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, q.device)
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    _, h_idx, d_idx = q_idx.shape
    prefix_blocks = _prefill_args(q_idx, w, k_idx, k_pooled_prefix, r, lk)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if plan is None:
        plan = PrefillPlan(lq, lk, hq, hkv, d, h_idx, d_idx, budget, r=r, row_chunk=row_chunk,
                           device=q.device)
    keep, pp = _pe_arg(pe)
    _call("qsa_prefill_forward", lq, lk, q_pos0, hq, hkv, d, h_idx, d_idx, r, budget, _ptr(q),
          _ptr(k), _ptr(v), _ptr(q_idx), _ptr(w), _ptr(k_idx), prefix_blocks * r,
          _ptr(k_pooled_prefix), _ptr(plan.k_pooled), scale, _ptr(plan.sel), _ptr(plan.out),
          _ptr(plan.lse), plan.row_chunk, _ptr(plan.ws), plan.ws_bytes, pp, _stream(q))
    del keep
    return plan.out, plan.lse, plan.sel, plan.k_pooled


def _bounds(cu_q: torch.Tensor, cu_k: torch.Tensor, max_lq, max_lk):
    """Host upper bounds of the sequence lengths; read from the device (a synchronising
    copy) only when the caller gives none."""
    if max_lq is None or max_lk is None:
        lq = (cu_q[1:] - cu_q[:-1]).max().item() if cu_q.numel() > 1 else 0
        lk = (cu_k[1:] - cu_k[:-1]).max().item() if cu_k.numel() > 1 else 0
        max_lq = lq if max_lq is None else max_lq
        max_lk = lk if max_lk is None else max_lk
    return int(max_lq), int(max_lk)


class VarlenPlan:
    """Outputs and workspace for packed (THD) prefill batches within given bounds."""

    def __init__(self, batch, total_q, max_lq, max_lk, hq, d, d_idx, budget, *, r=4,
                 row_chunk=None, device="cuda"):
        dev = torch.device(device)
        # about 16K score rows per selection chunk, whatever the batch
        self.row_chunk = row_chunk if row_chunk else max(64, 16384 // max(batch, 1))
        self.shape = (batch, total_q, max_lq, max_lk, budget, r)
        self.sel = torch.empty((total_q, budget // r), dtype=torch.int32, device=dev)
        self.out = torch.empty((total_q, hq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((total_q, hq), dtype=torch.float32, device=dev)
        self.k_pooled = torch.empty((batch, max_lk // r, d_idx), dtype=torch.bfloat16,
                                    device=dev)
        nbytes = _lib.load().qsa_prefill_varlen_workspace_bytes(batch, max_lq, max_lk, r, budget,
                                                                self.row_chunk)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        self.ws_bytes = nbytes


def qsa_prefill_varlen_forward(q, k, v, q_idx, w, k_idx, cu_seqlens_q, cu_seqlens_k, *,
                               budget: int, max_lq: Optional[int] = None,
                               max_lk: Optional[int] = None, scale: Optional[float] = None,
                               r: int = 4, row_chunk: Optional[int] = None,
                               plan: Optional[VarlenPlan] = None, pe=None):
    """Whole prefill of a packed batch. q [Tq,Hq,d], k/v [Tk,Hkv,d], q_idx [Tq,H_I,d_I],
    w [Tq,H_I], k_idx [Tk,d_I]; cu_seqlens_q/k int32 [B+1] on the device. Each sequence's
    queries are its last tokens. Returns (out, lse, sel with per-sequence block ids,
    k_pooled [B, max_lk/r, d_I])."""
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("q_idx", q_idx, torch.bfloat16),
                        ("w", w, torch.float32), ("k_idx", k_idx, torch.bfloat16),
                        ("cu_seqlens_q", cu_seqlens_q, torch.int32),
                        ("cu_seqlens_k", cu_seqlens_k, torch.int32)):
        _need(t, name, dt, q.device)
    batch = cu_seqlens_q.numel() - 1
    total_q, hq, d = q.shape
    _, hkv, _ = k.shape
    _, h_idx, d_idx = q_idx.shape
    max_lq, max_lk = _bounds(cu_seqlens_q, cu_seqlens_k, max_lq, max_lk)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if plan is None:
        plan = VarlenPlan(batch, total_q, max_lq, max_lk, hq, d, d_idx, budget, r=r,
                          row_chunk=row_chunk, device=q.device)
    keep, pp = _pe_arg(pe)
    _call("qsa_prefill_varlen_forward", batch, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), total_q,
          max_lq, max_lk, hq, hkv, d, h_idx, d_idx, r, budget, _ptr(q), _ptr(k), _ptr(v),
          _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(plan.k_pooled), scale, _ptr(plan.sel),
          _ptr(plan.out), _ptr(plan.lse), plan.row_chunk, _ptr(plan.ws), plan.ws_bytes,
          pp, _stream(q))
    del keep
    return plan.out, plan.lse, plan.sel, plan.k_pooled


def qsa_sparse_attn_varlen_fwd(q, k, v, sel, cu_seqlens_q, cu_seqlens_k, *,
                               scale: Optional[float] = None, r: int = 4,
                               out: Optional[torch.Tensor] = None,
                               lse: Optional[torch.Tensor] = None, max_lk: int = 0):
    """Attention of a packed batch over per-sequence selections sel [Tq, n_sel].
    max_lk: the longest sequence's key count if known (0: unknown), which only
    chooses the launch order."""
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("sel", sel, torch.int32),
                        ("cu_seqlens_q", cu_seqlens_q, torch.int32),
                        ("cu_seqlens_k", cu_seqlens_k, torch.int32)):
        _need(t, name, dt, q.device)
    total_q, hq, d = q.shape
    _, hkv, _ = k.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _call("qsa_sparse_attn_varlen_fwd", cu_seqlens_q.numel() - 1, _ptr(cu_seqlens_q),
          _ptr(cu_seqlens_k), total_q, max_lk, hq, hkv, d, r, sel.shape[1], _ptr(q), _ptr(k),
          _ptr(v), _ptr(sel), scale, _ptr(out), _ptr(lse), _stream(q))
    return out, lse


class DecodePlan:
    """Preallocated outputs and workspace for repeated decode steps of one shape."""

    def __init__(self, batch, hq, d, lmax, budget, *, r=4, device="cuda"):
        dev = torch.device(device)
        self.sel = torch.empty((batch, budget // r), dtype=torch.int32, device=dev)
        self.out = torch.empty((batch, hq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
        nbytes = _lib.load().qsa_decode_workspace_bytes(batch, hq, d, lmax, r, budget)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        self.ws_bytes = nbytes


def qsa_decode_forward(q, q_idx, w, k_pooled, k_cache, v_cache, seq_lens, *, budget: int,
                       scale: Optional[float] = None, r: int = 4,
                       plan: Optional[DecodePlan] = None):
    """Whole decode step. q [B,Hq,d], q_idx [B,H_I,d_I] (or [B,1,H_I,d_I]), w [B,H_I],
    k_pooled [B,Lmax/r,d_I], caches [B,Lmax,Hkv,d], seq_lens [B] int32.
    Returns (out, lse, sel)."""
    q_idx = q_idx.reshape(q_idx.shape[0], q_idx.shape[-2], q_idx.shape[-1])
    w = w.reshape(w.shape[0], w.shape[-1])
    for name, t, dt in (("q", q, torch.bfloat16), ("q_idx", q_idx, torch.bfloat16),
                        ("w", w, torch.float32), ("k_pooled", k_pooled, torch.bfloat16),
                        ("k_cache", k_cache, torch.bfloat16), ("v_cache", v_cache, torch.bfloat16),
                        ("seq_lens", seq_lens, torch.int32)):
        _need(t, name, dt, q.device)
    bsz, hq, d = q.shape
    _, lmax, hkv, _ = k_cache.shape
    _, h_idx, d_idx = q_idx.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if plan is None:
        plan = DecodePlan(bsz, hq, d, lmax, budget, r=r, device=q.device)
    _call("qsa_decode_forward", bsz, hq, hkv, d, h_idx, d_idx, r, budget, _ptr(q), _ptr(q_idx),
          _ptr(w), _ptr(k_pooled), k_pooled.stride(0), _ptr(k_cache), _ptr(v_cache),
          k_cache.stride(0), lmax, _ptr(seq_lens), scale, _ptr(plan.sel), _ptr(plan.out),
          _ptr(plan.lse), _ptr(plan.ws), plan.ws_bytes, _stream(q))
    return plan.out, plan.lse, plan.sel


def qsa_decode_forward_noalloc(q, q_idx, w, k_pooled, k_cache, v_cache, seq_lens, *,
                               budget: int, scale: Optional[float] = None, r: int = 4,
                               sel: Optional[torch.Tensor] = None,
                               out: Optional[torch.Tensor] = None,
                               lse: Optional[torch.Tensor] = None):
    """qsa_decode_forward without a workspace: the library's static device scratch
    serves instead (calls overlapping on one GPU race). Outputs are the caller's
    (allocated here when not given). Returns (out, lse, sel)."""
    q_idx = q_idx.reshape(q_idx.shape[0], q_idx.shape[-2], q_idx.shape[-1])
    w = w.reshape(w.shape[0], w.shape[-1])
    for name, t, dt in (("q", q, torch.bfloat16), ("q_idx", q_idx, torch.bfloat16),
                        ("w", w, torch.float32), ("k_pooled", k_pooled, torch.bfloat16),
                        ("k_cache", k_cache, torch.bfloat16), ("v_cache", v_cache, torch.bfloat16),
                        ("seq_lens", seq_lens, torch.int32)):
        _need(t, name, dt, q.device)
    bsz, hq, d = q.shape
    _, lmax, hkv, _ = k_cache.shape
    _, h_idx, d_idx = q_idx.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    sel = torch.empty((bsz, budget // r), dtype=torch.int32, device=q.device) if sel is None else sel
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _call("qsa_decode_forward_noalloc", bsz, hq, hkv, d, h_idx, d_idx, r, budget, _ptr(q),
          _ptr(q_idx), _ptr(w), _ptr(k_pooled), k_pooled.stride(0), _ptr(k_cache),
          _ptr(v_cache), k_cache.stride(0), lmax, _ptr(seq_lens), scale, _ptr(sel), _ptr(out),
          _ptr(lse), _stream(q))
    return out, lse, sel


def qsa_decode_forward_paged(q, q_idx, w, k_pooled, k_pool, v_pool, block_table, seq_lens, *,
                             budget: int, page_size: int, lmax: Optional[int] = None,
                             scale: Optional[float] = None, r: int = 4,
                             plan: Optional[DecodePlan] = None):
    """Whole decode step over a paged K/V cache. k_pool/v_pool [num_pages*page_size,Hkv,d],
    block_table int32 [B, pages per sequence] (page ids), k_pooled [B,Lmax/r,d_I];
    lmax defaults to page_size * block_table.shape[1]. Returns (out, lse, sel)."""
    q_idx = q_idx.reshape(q_idx.shape[0], q_idx.shape[-2], q_idx.shape[-1])
    w = w.reshape(w.shape[0], w.shape[-1])
    for name, t, dt in (("q", q, torch.bfloat16), ("q_idx", q_idx, torch.bfloat16),
                        ("w", w, torch.float32), ("k_pooled", k_pooled, torch.bfloat16),
                        ("k_pool", k_pool, torch.bfloat16), ("v_pool", v_pool, torch.bfloat16),
                        ("block_table", block_table, torch.int32),
                        ("seq_lens", seq_lens, torch.int32)):
        _need(t, name, dt, q.device)
    bsz, hq, d = q.shape
    slots, hkv, _ = k_pool.shape
    _, h_idx, d_idx = q_idx.shape
    lmax = page_size * block_table.shape[1] if lmax is None else lmax
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if plan is None:
        plan = DecodePlan(bsz, hq, d, lmax, budget, r=r, device=q.device)
    _call("qsa_decode_forward_paged", bsz, hq, hkv, d, h_idx, d_idx, r, budget, _ptr(q),
          _ptr(q_idx), _ptr(w), _ptr(k_pooled), k_pooled.stride(0), _ptr(k_pool), _ptr(v_pool),
          slots // page_size, page_size, _ptr(block_table), block_table.stride(0), lmax,
          _ptr(seq_lens), scale, _ptr(plan.sel), _ptr(plan.out), _ptr(plan.lse), _ptr(plan.ws),
          plan.ws_bytes, _stream(q))
    return plan.out, plan.lse, plan.sel
