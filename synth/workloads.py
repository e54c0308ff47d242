"""Workload definitions and the seeded generator of their inputs.

Recipe (the same for every workload; the sizes differ):

* q, k, v are drawn N(0, 1) and scaled by 1/sqrt(d) (d = attention head dim);
  the indexer queries and keys are drawn N(0, 1) and scaled by 1/sqrt(d_I).
  Every tensor is rounded once to bf16 (round to nearest even).
* The per-(token, head) indexer weights are U(0, 1) in fp32.
* Pooled indexer keys that arrive as a cache (the decode cache and the prefix of a
  chunked prefill) are drawn directly, N(0, 1)/sqrt(d_I) in bf16.
* Needles: with spacing S, n = Lk // S needles; needle i sits at block
  i*S/r + U{0, S/r - 1} and every indexer key of that block is bf16(u_i) with
  u_i a random unit vector, so the block's mean-pooled key is exactly u_i.
  10% of the query rows that have at least one needle strictly before their own
  block get aligned with one of those needles chosen uniformly: every indexer head
  of the row becomes bf16(u_i * |original row|).

Every tensor has its own child of ``numpy.random.SeedSequence(seed)`` and large
tensors are drawn in row chunks with one grandchild seed per chunk, so any chunk
can be regenerated alone. Values come from torch's generator on the requested
device; the same seed gives different numbers on the CPU and on the GPU (both
follow the recipe above), so a parity test draws once and copies to the host.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

# Rows drawn per seeded chunk (a chunk is the unit that can be regenerated alone).
CHUNK_ELEMS = 1 << 24


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill" or "decode"
    batch: int
    lq: int  # query tokens per sequence
    lk: int  # key tokens per sequence, including the new ones
    q_pos0: int  # absolute position of query row 0 (prefill)
    hq: int
    hkv: int
    d: int
    h_i: int
    d_i: int
    r: int
    budget: int
    seed: int
    needle_spacing: int  # 0: no needles
    pooled_prefix_blocks: int  # leading blocks whose pooled keys arrive as a cache
    aligned_fraction: float = 0.10
    smooth: int = 0  # prefill: > 0 correlates q_idx and w along the tokens over ~smooth tokens

    @property
    def n_sel(self) -> int:
        return self.budget // self.r

    @property
    def nblk(self) -> int:
        return self.lk // self.r

    @property
    def pooled_from_tokens(self) -> int:
        """First token whose indexer key is given raw (to be pooled)."""
        return self.pooled_prefix_blocks * self.r


CONFIGS: Dict[str, Workload] = {
    # 1 sequence, L=2048, 4 query heads / 1 KV head at d=128, indexer 4x64, K=256.
    "tiny": Workload("tiny", "prefill", 1, 2048, 2048, 0, 4, 1, 128, 4, 64, 4, 256, 0, 256, 0),
    # Model shape at 32K: 24/2 heads, d=256, indexer 4x128, K=2048, needle per 1024 tokens.
    "prefill32k": Workload("prefill32k", "prefill", 1, 32768, 32768, 0, 24, 2, 256, 4, 128, 4,
                           2048, 1, 1024, 0),
    # Long prefill at 128K, needle per 4096 tokens.
    "prefill128k": Workload("prefill128k", "prefill", 1, 131072, 131072, 0, 24, 2, 256, 4, 128,
                            4, 2048, 2, 4096, 0),
    # Decode: 8 sequences, one new token each, 1M-token caches (K/V and pooled keys).
    "decode1m": Workload("decode1m", "decode", 8, 1, 1048576, 1048575, 24, 2, 256, 4, 128, 4,
                         2048, 3, 0, 262144),
    # Chunked prefill: 8192 new tokens on a cached prefix of 1,040,384 tokens.
    "chunked1m": Workload("chunked1m", "prefill", 1, 8192, 1048576, 1040384, 24, 2, 256, 4, 128,
                          4, 2048, 4, 16384, 1040384 // 4),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with some fields replaced (smaller test shapes)."""
    return dataclasses.replace(CONFIGS[name], **overrides)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a bf16 tensor as a host uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


_TENSORS = ("q", "k", "v", "q_idx", "k_idx", "w", "needles", "k_pooled")


def _child_seeds(seed: int) -> Dict[str, np.random.SeedSequence]:
    kids = np.random.SeedSequence(seed).spawn(len(_TENSORS))
    return dict(zip(_TENSORS, kids))


def _chunk_seed(ss: np.random.SeedSequence, chunk: int) -> int:
    child = np.random.SeedSequence(entropy=ss.entropy, spawn_key=ss.spawn_key + (chunk,))
    return int(child.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _fill_normal(out: torch.Tensor, ss: np.random.SeedSequence, scale: float) -> None:
    """Fill a bf16 tensor with bf16(N(0,1) * scale), one seeded draw per row chunk."""
    if out.numel() == 0:
        return
    flat = out.view(out.shape[0], -1) if out.dim() > 1 else out.view(1, -1)
    rows, cols = flat.shape
    rows_per_chunk = max(1, CHUNK_ELEMS // max(cols, 1))
    gen = torch.Generator(device=out.device)
    for c, r0 in enumerate(range(0, rows, rows_per_chunk)):
        r1 = min(rows, r0 + rows_per_chunk)
        gen.manual_seed(_chunk_seed(ss, c))
        x = torch.randn((r1 - r0, cols), generator=gen, device=out.device, dtype=torch.float32)
        x.mul_(scale)
        flat[r0:r1].copy_(x)  # fp32 -> bf16 rounds to nearest even


def _smoothed_normal(shape, ss: np.random.SeedSequence, span: int, device) -> torch.Tensor:
    """fp32 draws with N(0, 1) marginals, correlated along axis 0: white N(0, 1) noise
    filtered by a causal exponential window (weights a^k, a = 1 - 1/span, k < 4 span),
    normalised to unit variance; the lag-l correlation is about a^l."""
    gen = torch.Generator(device=device)
    gen.manual_seed(_chunk_seed(ss, 0))
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    a = 1.0 - 1.0 / span
    taps = 4 * span
    kern = a ** torch.arange(taps, device=device, dtype=torch.float32)
    kern = kern / kern.square().sum().sqrt()
    flat = x.reshape(shape[0], -1).T.unsqueeze(1)  # [channels, 1, tokens]
    y = torch.nn.functional.conv1d(torch.nn.functional.pad(flat, (taps - 1, 0)),
                                   kern.flip(0).view(1, 1, taps))
    return y.squeeze(1).T.reshape(shape)


def _fill_uniform(out: torch.Tensor, ss: np.random.SeedSequence) -> None:
    gen = torch.Generator(device=out.device)
    gen.manual_seed(_chunk_seed(ss, 0))
    out.copy_(torch.rand(out.shape, generator=gen, device=out.device, dtype=torch.float32))


def _plant_needles(wl: Workload, ss: np.random.SeedSequence, q_idx: torch.Tensor,
                   k_idx: Optional[torch.Tensor], k_pooled: Optional[torch.Tensor]) -> dict:
    """Plant needle blocks and align a fraction of the query rows with them."""
    r = wl.r
    n = wl.lk // wl.needle_spacing
    seg_blocks = wl.needle_spacing // r
    rng = np.random.default_rng(ss)
    blocks = np.arange(n, dtype=np.int64) * seg_blocks + rng.integers(0, seg_blocks, size=n)
    g = rng.standard_normal((n, wl.d_i))
    u = g / np.linalg.norm(g, axis=1, keepdims=True)
    u_bf = torch.from_numpy(u.astype(np.float32)).to(torch.bfloat16)
    dev = q_idx.device
    for i, b in enumerate(blocks.tolist()):
        if b < wl.pooled_prefix_blocks:
            k_pooled[b] = u_bf[i].to(dev)
        else:
            t0 = b * r - wl.pooled_from_tokens
            k_idx[t0:t0 + r] = u_bf[i].to(dev).unsqueeze(0).expand(r, -1)
    # Rows whose own block has at least one needle strictly before it.
    pos = wl.q_pos0 + np.arange(wl.lq, dtype=np.int64)
    own = pos // r
    n_before = np.searchsorted(blocks, own, side="left")  # blocks is increasing
    eligible = np.nonzero(n_before > 0)[0]
    n_aligned = min(len(eligible), int(round(wl.aligned_fraction * wl.lq)))
    rows = np.sort(rng.choice(eligible, size=n_aligned, replace=False)) if n_aligned else \
        np.zeros(0, dtype=np.int64)
    which = np.array([rng.integers(0, n_before[i]) for i in rows], dtype=np.int64)
    if n_aligned:
        rows_t = torch.from_numpy(rows).to(dev)
        orig = q_idx[rows_t].float()  # [n, H_I, d_I]
        norms = orig.norm(dim=-1, keepdim=True)  # [n, H_I, 1]
        dirs = u_bf[torch.from_numpy(which)].float().to(dev).unsqueeze(1)  # [n, 1, d_I]
        q_idx[rows_t] = (dirs * norms).to(torch.bfloat16)
    return {
        "needle_blocks": blocks,
        "aligned_rows": rows.astype(np.int64),
        "aligned_blocks": blocks[which] if n_aligned else np.zeros(0, dtype=np.int64),
    }


def generate(wl: Workload, device="cpu", seq_lens=None) -> dict:
    """Draw every input of a workload on ``device``.

    Prefill returns q [Lq,Hq,d], k/v [Lk,Hkv,d], q_idx [Lq,H_I,d_I], w [Lq,H_I],
    k_idx [Lk - prefix_tokens, d_I] (the raw indexer keys still to be pooled) and,
    when the workload has a pooled prefix, k_pooled_prefix [prefix_blocks, d_I].
    Decode returns q [B,Hq,d], k_cache/v_cache [B,Lk,Hkv,d], q_idx [B,1,H_I,d_I],
    w [B,1,H_I], k_pooled [B,Lk//r,d_I] and seq_lens [B] (int32).
    """
    device = torch.device(device)
    seeds = _child_seeds(wl.seed)
    bf = torch.bfloat16
    sd, sdi = 1.0 / math.sqrt(wl.d), 1.0 / math.sqrt(wl.d_i)
    out: dict = {"workload": wl}
    if wl.kind == "prefill":
        q = torch.empty((wl.lq, wl.hq, wl.d), dtype=bf, device=device)
        k = torch.empty((wl.lk, wl.hkv, wl.d), dtype=bf, device=device)
        v = torch.empty((wl.lk, wl.hkv, wl.d), dtype=bf, device=device)
        q_idx = torch.empty((wl.lq, wl.h_i, wl.d_i), dtype=bf, device=device)
        k_idx = torch.empty((wl.lk - wl.pooled_from_tokens, wl.d_i), dtype=bf, device=device)
        w = torch.empty((wl.lq, wl.h_i), dtype=torch.float32, device=device)
        _fill_normal(q, seeds["q"], sd)
        _fill_normal(k, seeds["k"], sd)
        _fill_normal(v, seeds["v"], sd)
        _fill_normal(k_idx, seeds["k_idx"], sdi)
        if wl.smooth:
            # Neighbouring queries alike (real selections overlap): the same marginals,
            # correlated along the tokens; w through the normal CDF stays U(0, 1).
            q_idx.copy_(_smoothed_normal(q_idx.shape, seeds["q_idx"], wl.smooth, device) * sdi)
            z = _smoothed_normal(w.shape, seeds["w"], wl.smooth, device)
            w.copy_(0.5 * (1.0 + torch.erf(z / math.sqrt(2.0))))
        else:
            _fill_normal(q_idx, seeds["q_idx"], sdi)
            _fill_uniform(w, seeds["w"])
        kp = None
        if wl.pooled_prefix_blocks:
            kp = torch.empty((wl.pooled_prefix_blocks, wl.d_i), dtype=bf, device=device)
            _fill_normal(kp, seeds["k_pooled"], sdi)
        out.update(q=q, k=k, v=v, q_idx=q_idx, k_idx=k_idx, w=w, k_pooled_prefix=kp)
        if wl.needle_spacing:
            out.update(_plant_needles(wl, seeds["needles"], q_idx, k_idx, kp))
        else:
            out.update(needle_blocks=np.zeros(0, np.int64), aligned_rows=np.zeros(0, np.int64),
                       aligned_blocks=np.zeros(0, np.int64))
        return out
    if wl.kind != "decode":
        raise ValueError(f"unknown workload kind {wl.kind!r}")
    b = wl.batch
    q = torch.empty((b, wl.hq, wl.d), dtype=bf, device=device)
    kc = torch.empty((b, wl.lk, wl.hkv, wl.d), dtype=bf, device=device)
    vc = torch.empty((b, wl.lk, wl.hkv, wl.d), dtype=bf, device=device)
    q_idx = torch.empty((b, 1, wl.h_i, wl.d_i), dtype=bf, device=device)
    w = torch.empty((b, 1, wl.h_i), dtype=torch.float32, device=device)
    kp = torch.empty((b, wl.lk // wl.r, wl.d_i), dtype=bf, device=device)
    _fill_normal(q, seeds["q"], sd)
    _fill_normal(kc.view(b * wl.lk, -1), seeds["k"], sd)
    _fill_normal(vc.view(b * wl.lk, -1), seeds["v"], sd)
    _fill_normal(q_idx, seeds["q_idx"], sdi)
    _fill_uniform(w, seeds["w"])
    _fill_normal(kp.view(b * (wl.lk // wl.r), -1), seeds["k_pooled"], sdi)
    if seq_lens is None:
        seq_lens = [wl.lk] * b
    sl = torch.tensor(list(seq_lens), dtype=torch.int32, device=device)
    out.update(q=q, k_cache=kc, v_cache=vc, q_idx=q_idx, w=w, k_pooled=kp, seq_lens=sl)
    return out


def serving_lengths(n_seqs: int, total: int, lo: int, seed: int) -> list:
    """A seeded length mix for a packed prefill batch: n_seqs lengths, each at least
    ``lo``, summing to ``total``: Dirichlet(1, ..., 1) shares of the tokens above the
    floor, rounded down, the remainder given to the last sequence."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    share = rng.dirichlet(np.ones(n_seqs))
    extra = np.floor(share * (total - n_seqs * lo)).astype(np.int64)
    lens = lo + extra
    lens[-1] += total - int(lens.sum())
    return [int(x) for x in lens]


def generate_varlen(wl: Workload, lens, device="cpu") -> dict:
    """Draw a packed (THD) batch: sequence b has lens[b] = (lq_b, lk_b), its queries
    being its last lq_b tokens. Each sequence is drawn by ``generate`` as a prefill
    workload of its own shapes (seed wl.seed * 1000 + b, no pooled prefix), and the
    tensors are concatenated along the token axis. Returns q, k, v, q_idx, w, k_idx,
    cu_q and cu_k (int32, on ``device``), the lengths, and each sequence's needle
    rows as packed row indices."""
    parts = []
    for b, (lq, lk) in enumerate(lens):
        wb = dataclasses.replace(wl, kind="prefill", batch=1, lq=int(lq), lk=int(lk),
                                 q_pos0=int(lk) - int(lq), seed=wl.seed * 1000 + b,
                                 pooled_prefix_blocks=0,
                                 needle_spacing=(wl.needle_spacing
                                                 if wl.needle_spacing and lk >= wl.needle_spacing
                                                 else 0))
        parts.append(generate(wb, device=device))
    cu_q = np.concatenate([[0], np.cumsum([lq for lq, _ in lens])]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum([lk for _, lk in lens])]).astype(np.int32)
    out = {name: torch.cat([p[name] for p in parts], dim=0)
           for name in ("q", "k", "v", "q_idx", "w", "k_idx")}
    out["cu_q"] = torch.from_numpy(cu_q).to(device)
    out["cu_k"] = torch.from_numpy(cu_k).to(device)
    out["lens"] = [(int(a), int(b)) for a, b in lens]
    out["aligned_rows"] = np.concatenate(
        [p["aligned_rows"] + cu_q[b] for b, p in enumerate(parts)]).astype(np.int64)
    out["aligned_blocks"] = np.concatenate([p["aligned_blocks"] for p in parts]).astype(np.int64)
    return out


def decode_query_sets(wl: Workload, n_sets: int, device="cpu") -> list:
    """n_sets further draws of a decode workload's new-token inputs (q [B,Hq,d],
    q_idx [B,1,H_I,d_I], w [B,1,H_I]) by the same recipe, set i from the seed
    sequence (wl.seed, 1000 + i): successive decode steps then score, select and
    gather different blocks of the same caches."""
    assert wl.kind == "decode"
    device = torch.device(device)
    b, bf = wl.batch, torch.bfloat16
    sets = []
    for i in range(n_sets):
        kids = dict(zip(("q", "q_idx", "w"),
                        np.random.SeedSequence([wl.seed, 1000 + i]).spawn(3)))
        q = torch.empty((b, wl.hq, wl.d), dtype=bf, device=device)
        q_idx = torch.empty((b, 1, wl.h_i, wl.d_i), dtype=bf, device=device)
        w = torch.empty((b, 1, wl.h_i), dtype=torch.float32, device=device)
        _fill_normal(q, kids["q"], 1.0 / math.sqrt(wl.d))
        _fill_normal(q_idx, kids["q_idx"], 1.0 / math.sqrt(wl.d_i))
        _fill_uniform(w, kids["w"])
        sets.append({"q": q, "q_idx": q_idx, "w": w})
    return sets

