#!/usr/bin/env python3
"""Throughput of the QSA forward path on one MI355X.

One step is one pass of the whole prefill path over the 128K-token workload
(1 sequence, 24 query heads / 2 KV groups at d=256, indexer 4 heads x 128, r=4,
budget 2048): pool the indexer keys, score every causal block, keep the top
blocks, attend over the kept tokens. Inputs are seeded synthetic tensors already
resident in HBM. The line also reports the 1M-context decode step (8 sequences,
one new token each) and the oracle's CPU throughput on a bounded sample.

Prints ONE JSON line. Only one GPU is supported.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

METRIC = "QSA fwd tokens/s: 128K prefill & 1M-ctx decode; % MFMA / HBM roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="prefill128k",
                   choices=["prefill128k", "prefill32k", "chunked1m", "tiny"])
    p.add_argument("--row-chunk", type=int, default=65536)
    p.add_argument("--select", choices=["auto", "fused", "plain"], default="auto",
                   help="selection path of the step: the fused score/top-k, the two-kernel "
                        "one (scores materialised, then top-k), or the library's default for "
                        "the workload (auto)")
    p.add_argument("--decode-steps", type=int, default=50)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-backward", action="store_true",
                   help="skip the sparse-attention backward measurement")
    p.add_argument("--no-warmup", action="store_true",
                   help="skip the indexer KL warm-up measurement")
    p.add_argument("--no-paged", action="store_true",
                   help="skip the decode step over a paged K/V cache")
    p.add_argument("--no-varlen", action="store_true",
                   help="skip the packed variable-length prefill batch")
    p.add_argument("--no-other", action="store_true",
                   help="skip the 32K and chunked-1M prefill steps")
    p.add_argument("--no-tile", action="store_true",
                   help="skip the multi-row attention tile measurement")
    p.add_argument("--tile-only", choices=["random", "correlated"], default=None,
                   help="only select and run the attention on the workload (correlated: "
                        "smooth 100 indexer inputs), one per-row call and one tile call with "
                        "the union always taken, each after one warm-up call (a short run "
                        "for the profiler's counters) and exit")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB three times (scale for the "
                        "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


def copy_calibration(torch, mib):
    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "launches": 3}), flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
COUNTERS = os.path.join(ROOT, "profiles", "sparse_attn_prefill128k_counters.md")
ATTN_SOURCES = [os.path.join(ROOT, "block_sparse_attention_06_amd", "csrc", f)
                for f in ("attention.hip", "attn_step.h", "qsa_device.h")]


def attention_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def progress(msg):
    """One line on stderr per finished phase (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def counted_traffic():
    """HBM bytes of one attention call over all rows (all its launches) from the
    committed counter summary, or None when the summary is missing or was taken on a
    different attention kernel source."""
    import re
    try:
        with open(COUNTERS) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_call=(\d+) kernel_source=([0-9a-f]+)", text)
    if not m or m.group(2) != attention_source_hash():
        return None
    return int(m.group(1))


def gather_ceiling(torch, Q, dev, mib, sequential, n_waves=65536, steps=32):
    """GB/s of the library's gather probe: 4 KiB blocks, the attention step's pattern."""
    buf = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    nblk = (mib << 20) // 4096
    n_ids = n_waves * steps * 4
    if sequential:
        ids = (torch.arange(n_ids, device=dev, dtype=torch.int64) % nblk).to(torch.int32)
    else:
        g = torch.Generator(device=dev)
        g.manual_seed(7)
        ids = torch.randint(0, nblk, (n_ids,), generator=g, device=dev, dtype=torch.int32)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    from block_sparse_attention_06_amd.probe import probe_gather
    probe_gather(buf, ids, steps, sink)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(3)]
    for a, b in evs:
        a.record()
        probe_gather(buf, ids, steps, sink)
        b.record()
    torch.cuda.synchronize()
    ms = min(a.elapsed_time(b) for a, b in evs)
    del buf, ids
    return n_waves * steps * 16384 / (ms * 1e-3) / 1e9


def write_ceiling(torch, dev, nbytes, nontemporal, reps=3):
    """GB/s of the probe library's write stream (16-byte stores, 1 KiB per wave
    instruction: the score GEMM's store pattern) over a buffer of nbytes."""
    from block_sparse_attention_06_amd.probe import probe_write
    buf = torch.empty(nbytes // 16 * 16, dtype=torch.uint8, device=dev)
    probe_write(buf, nontemporal)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record()
        probe_write(buf, nontemporal)
        b.record()
    torch.cuda.synchronize()
    ms = min(a.elapsed_time(b) for a, b in evs)
    n = buf.numel()
    del buf
    return n / (ms * 1e-3) / 1e9


def score_write_bytes(wl):
    """fp32 scores the score GEMM stores in a step: each row its min(own block, n_blocks)
    candidates, rounded up to the 4 of one 16-byte store."""
    import numpy as np
    t = wl.q_pos0 + np.arange(wl.lq, dtype=np.int64)
    lim = np.minimum(t // wl.r, wl.lk // wl.r)
    return int(((lim + 3) // 4 * 16).sum())


def kept_tokens(t, n_sel, r=4):
    """Tokens attended by a query at position t (array) under a full selection."""
    own = t // r
    kept_blocks = (own + 1).clip(max=n_sel)
    return r * (kept_blocks - 1) + (t - r * own) + 1


def attention_bytes(wl, t):
    """Algorithmic bytes of one attention launch: gathered K/V, q, out, sel, lse."""
    gathered = int(kept_tokens(t, wl.n_sel).sum()) * wl.hkv * 2 * wl.d * 2
    per_row = wl.hq * wl.d * 2 * 2 + wl.n_sel * 4 + wl.hq * 4
    return gathered + len(t) * per_row


def attention_flops(wl, t):
    """Algorithmic flops of the attention over the kept tokens: per (row, head, kept
    token) a d-long dot product for the score and a d-long P.V update, 2 flop per
    multiply-add each."""
    return int(kept_tokens(t, wl.n_sel).sum()) * wl.hq * wl.d * 4


def score_flops(wl, t):
    """Algorithmic flops of the indexer score GEMM (2 * H_I * d_I per scored block)."""
    own = (t // wl.r).clip(max=wl.nblk)
    return int(own.sum()) * 2 * wl.h_i * wl.d_i


def select_path(Q, wl, select):
    """'fused' or 'plain' for a --select choice on a workload."""
    if select == "auto":
        return "fused" if Q.prefer_fused_select(wl.lk, wl.r) else "plain"
    return select


def bench_prefill(args, torch, Q, wl, inp, fused=None):
    dev = inp["q"].device
    fused = (select_path(Q, wl, args.select) == "fused") if fused is None else fused
    plan = Q.PrefillPlan(wl.lq, wl.lk, wl.hq, wl.hkv, wl.d, wl.h_i, wl.d_i, wl.budget,
                         row_chunk=args.row_chunk, device=dev, fused=fused)
    scale = 1.0 / math.sqrt(wl.d)

    def step(ev_s=None, ev_a=None, ev_b=None):
        if ev_s is not None:
            ev_s.record()
        Q.qsa_prefill_select(inp["q_idx"], inp["w"], inp["k_idx"], lk=wl.lk, budget=wl.budget,
                             q_pos0=wl.q_pos0, k_pooled_prefix=inp["k_pooled_prefix"], plan=plan)
        if ev_a is not None:
            ev_a.record()
        Q.qsa_sparse_attn_fwd(inp["q"], inp["k"], inp["v"], plan.sel, q_pos0=wl.q_pos0,
                              scale=scale, out=plan.out, lse=plan.lse)
        if ev_b is not None:
            ev_b.record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_, a, b in evs:
        step(s_, a, b)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = sum(a.elapsed_time(b) for _, a, b in evs) / len(evs)
    bench_prefill.step_ms = sorted(s_.elapsed_time(b) for s_, _, b in evs)
    return wall, attn_ms, plan


def bench_score_gemm(torch, Q, wl, inp, plan, row_chunk, reps=3):
    """The indexer score GEMM alone over the same row chunks as the step (pooled keys
    of the step's own pooling), into a chunk-sized scratch: ms per step's worth."""
    kp = plan.k_pooled
    nb_all = kp.shape[0]
    scratch = torch.empty(min(row_chunk, wl.lq) * Q.score_ld(nb_all), dtype=torch.float32,
                          device=kp.device)
    chunks = []
    for c0 in range(0, wl.lq, row_chunk):
        c1 = min(wl.lq, c0 + row_chunk)
        nb = min(nb_all, (wl.q_pos0 + c1 - 1) // wl.r)
        chunks.append((c0, c1, nb))

    def run():
        for c0, c1, nb in chunks:
            ld = Q.score_ld(nb)
            Q.qsa_index_scores(inp["q_idx"][c0:c1], inp["w"][c0:c1], kp, q_pos0=wl.q_pos0 + c0,
                               nblk=nb, out=scratch[: (c1 - c0) * ld].view(c1 - c0, ld))

    ms = time_calls(torch, run, reps) * 1e3
    del scratch
    return ms


def percentiles(xs):
    """p10 / p50 / p90 of a sorted list (nearest rank)."""
    n = len(xs)
    pick = lambda q: xs[min(n - 1, max(0, int(math.ceil(q * n)) - 1))]
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def bench_other_prefill(torch, Q, name, select, steps=5):
    """A whole prefill step (select + attention) on another workload: tokens/s, with
    the step's selection path and, for comparison, the other one."""
    import types
    from synth import generate, workload
    owl = workload(name)
    oinp = generate(owl, device="cuda")
    torch.cuda.synchronize()
    select = select_path(Q, owl, select)
    res = {"query_tokens": owl.lq, "context": owl.lk, "q_pos0": owl.q_pos0, "select": select}
    for path in (select, "plain" if select == "fused" else "fused"):
        args = types.SimpleNamespace(row_chunk=min(65536, owl.lq), warmup=1, steps=steps,
                                     select=path)
        wall, attn_ms, plan = bench_prefill(args, torch, Q, owl, oinp)
        step_ms = bench_prefill.step_ms
        del plan
        torch.cuda.empty_cache()
        if path == select:
            res.update({"tokens_per_s": owl.lq * steps / wall, "ms_per_step": wall / steps * 1e3,
                        "attention_ms": attn_ms, "step_ms": percentiles(step_ms),
                        "steps": steps})
        else:
            res[f"ms_per_step_{path}_select"] = wall / steps * 1e3
    del oinp
    torch.cuda.empty_cache()
    return res


def backward_bytes(wl, t):
    """Algorithmic bytes of one backward call over full selections at positions t.

    Query side: the kept K and V rows (as the forward), q, dout and out per row, sel,
    lse, dq and D. Key side: per (kept block, row) pair and KV group the row's q and
    dout for the group's heads plus lse and D, the pair itself (block and row, 8 B,
    written and read once), each key block's K and V, and dk, dv."""
    import numpy as np
    grp = wl.hq // wl.hkv
    gathered = int(kept_tokens(t, wl.n_sel).sum()) * wl.hkv * 2 * wl.d * 2
    per_row = wl.hq * wl.d * 2 * 3 + wl.n_sel * 4 + wl.hq * 4 * 2 + wl.hq * wl.d * 4
    pairs = int(np.minimum(t // wl.r + 1, wl.n_sel).sum())
    per_pair = wl.hkv * (2 * grp * wl.d * 2 + 2 * grp * 4) + 16
    keys = wl.lk * wl.hkv * wl.d * (2 * 2 + 2 * 4)
    return gathered + len(t) * per_row + pairs * per_pair + keys


def bench_backward(torch, Q, wl, inp, plan, reps=2):
    """Whole backward call (inverse selection, dq, dk/dv) on the forward's outputs."""
    g = torch.Generator(device=inp["q"].device)
    g.manual_seed(11)
    dout = torch.randn(inp["q"].shape, generator=g, device=inp["q"].device).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(wl.d)
    nbytes = Q.ops._lib.load().qsa_sparse_attn_bwd_workspace_bytes(wl.lq, wl.lk, wl.hq, wl.r,
                                                                   wl.n_sel)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=inp["q"].device)

    def run():
        return Q.qsa_sparse_attn_bwd(inp["q"], inp["k"], inp["v"], plan.sel, plan.out, plan.lse,
                                     dout, q_pos0=wl.q_pos0, scale=scale, workspace=ws)

    grads = run()
    del grads
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record()
        grads = run()
        b.record()
        del grads
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / reps
    del ws, dout
    return ms


def time_calls(torch, f, reps):
    """Average seconds of f() over reps calls after one untimed call (HIP events)."""
    f()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        f()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e-3


def bench_attention_tile(torch, Q, wl, inp, sel, reps=3):
    """The multi-row attention tile (qsa_sparse_attn_fwd_tiled) against the per-row
    kernel, on the step's own selections (random rows: neighbours share few blocks) and
    on the same workload with token-correlated indexer inputs (smooth 100: neighbours
    share most blocks): ms per call over all rows, the union always and chosen by the
    sampled overlap (32 of 64)."""
    import math
    from synth import generate, workload
    scale = 1.0 / math.sqrt(wl.d)
    res = {"what": "attention over all rows of the workload, ms per call"}

    def run(name, q, k, v, s):
        out = torch.empty_like(q)
        lse = torch.empty((q.shape[0], wl.hq), dtype=torch.float32, device=q.device)
        r = {"per_row_ms": 1e3 * time_calls(torch, lambda: Q.qsa_sparse_attn_fwd(
            q, k, v, s, q_pos0=wl.q_pos0, scale=scale, out=out, lse=lse), reps)}
        for key, ms in (("tile_union_ms", 0), ("tile_by_overlap_ms", 32)):
            r[key] = 1e3 * time_calls(torch, lambda: Q.qsa_sparse_attn_fwd_tiled(
                q, k, v, s, q_pos0=wl.q_pos0, scale=scale, min_shared=ms, out=out, lse=lse), reps)
        res[name] = r
        progress(f"attention tile ({name}): per row {r['per_row_ms']:.1f} ms, union "
                 f"{r['tile_union_ms']:.1f} ms, by overlap {r['tile_by_overlap_ms']:.1f} ms")

    run("random", inp["q"], inp["k"], inp["v"], sel)
    swl = workload(wl.name, smooth=100)
    sinp = generate(swl, device="cuda")
    ssel, _ = Q.qsa_prefill_select(sinp["q_idx"], sinp["w"], sinp["k_idx"], lk=swl.lk,
                                   budget=swl.budget, q_pos0=swl.q_pos0,
                                   k_pooled_prefix=sinp["k_pooled_prefix"], row_chunk=16384)
    run("correlated (smooth 100)", sinp["q"], sinp["k"], sinp["v"], ssel)
    del sinp, ssel
    torch.cuda.empty_cache()
    return res


def tile_only(torch, Q, name, kind):
    """--tile-only: the attention of one 128K-style workload, per row and as the tile
    (union always), one call each after a warm-up call; prints one JSON line."""
    import math
    from synth import generate, workload
    wl = workload(name, smooth=100) if kind == "correlated" else workload(name)
    inp = generate(wl, device="cuda")
    sel, _ = Q.qsa_prefill_select(inp["q_idx"], inp["w"], inp["k_idx"], lk=wl.lk,
                                  budget=wl.budget, q_pos0=wl.q_pos0,
                                  k_pooled_prefix=inp["k_pooled_prefix"], row_chunk=16384)
    scale = 1.0 / math.sqrt(wl.d)
    out = torch.empty_like(inp["q"])
    lse = torch.empty((wl.lq, wl.hq), dtype=torch.float32, device="cuda")
    per_row = time_calls(torch, lambda: Q.qsa_sparse_attn_fwd(
        inp["q"], inp["k"], inp["v"], sel, q_pos0=wl.q_pos0, scale=scale, out=out, lse=lse), 1)
    tile = time_calls(torch, lambda: Q.qsa_sparse_attn_fwd_tiled(
        inp["q"], inp["k"], inp["v"], sel, q_pos0=wl.q_pos0, scale=scale, min_shared=0,
        out=out, lse=lse), 1)
    print(json.dumps({"workload": wl.name, "selections": kind, "per_row_ms": per_row * 1e3,
                      "tile_union_ms": tile * 1e3}), flush=True)


def paged_copy(torch, kc, vc, page_size, seed=1):
    """The caches [B, L, Hkv, d] scattered into pools of shuffled pages (the layout a
    serving engine's page allocator leaves), and the block table."""
    bsz, L, hkv, d = kc.shape
    n_per = L // page_size
    g = torch.Generator(device="cpu").manual_seed(seed)
    table = torch.randperm(bsz * n_per, generator=g).view(bsz, n_per).to(torch.int32)
    table = table.to(kc.device)
    slots = (table.long()[:, :, None] * page_size
             + torch.arange(page_size, device=kc.device)).reshape(-1)
    pools = []
    for c in (kc, vc):
        pool = torch.empty((bsz * L, hkv, d), dtype=c.dtype, device=c.device)
        pool[slots] = c.reshape(-1, hkv, d)
        pools.append(pool)
    del slots
    return pools[0], pools[1], table


def bench_decode(args, torch, Q, wl, inp, paged=None, query_sets=None):
    """Seconds per decode step; with paged = (k_pool, v_pool, table, page_size) the
    step reads K/V through the block table. With query_sets, step i takes set
    i % len(query_sets) (new queries over the same caches), so that the blocks a step
    selects and gathers differ from the previous step's."""
    plan = Q.DecodePlan(wl.batch, wl.hq, wl.d, wl.lk, wl.budget, device=inp["q"].device)
    sets = query_sets or [{"q": inp["q"], "q_idx": inp["q_idx"], "w": inp["w"]}]

    def step(i):
        x = sets[i % len(sets)]
        if paged is None:
            Q.qsa_decode_forward(x["q"], x["q_idx"], x["w"], inp["k_pooled"],
                                 inp["k_cache"], inp["v_cache"], inp["seq_lens"],
                                 budget=wl.budget, plan=plan)
        else:
            Q.qsa_decode_forward_paged(x["q"], x["q_idx"], x["w"], inp["k_pooled"],
                                       paged[0], paged[1], paged[2], inp["seq_lens"],
                                       budget=wl.budget, page_size=paged[3], lmax=wl.lk,
                                       plan=plan)

    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.decode_steps):
        step(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / args.decode_steps


def bench_warmup(torch, Q, name="prefill32k", reps=2):
    """The indexer's KL warm-up on one workload: dense target (lse pass + pooled pass),
    indexer scores, KL loss with its score gradient, and the indexer's backward."""
    import numpy as np
    from synth import generate, workload
    wl = workload(name)
    inp = generate(wl, device="cuda")
    kp = Q.qsa_pool_keys(inp["k_idx"])
    scale = 1.0 / math.sqrt(wl.d)
    nblk = wl.lk // wl.r
    ev = {k: [] for k in ("target", "scores", "loss", "indexer_bwd")}
    for rep in range(reps + 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        e[0].record()
        lse, target = Q.qsa_indexer_kl_target(inp["q"], inp["k"], q_pos0=wl.q_pos0, scale=scale)
        e[1].record()
        scores = Q.qsa_index_scores(inp["q_idx"], inp["w"], kp, q_pos0=wl.q_pos0)
        e[2].record()
        loss, ds = Q.qsa_indexer_kl_loss(scores, target, nblk=nblk, q_pos0=wl.q_pos0)
        e[3].record()
        grads = Q.qsa_index_scores_bwd(inp["q_idx"], inp["w"], kp, ds, q_pos0=wl.q_pos0,
                                       n_tokens=wl.lk)
        e[4].record()
        torch.cuda.synchronize()
        if rep:
            for i, k in enumerate(ev):
                ev[k].append(e[i].elapsed_time(e[i + 1]))
        del lse, target, scores, loss, ds, grads
    ms = {k: sum(v) / len(v) for k, v in ev.items()}
    t = wl.q_pos0 + np.arange(wl.lq, dtype=np.int64)
    # dense passes: S = q.k over all causal keys, once for the lse and once for the
    # target (2 flop per multiply-add, every head)
    dense_flops = 2 * int((t + 1).sum()) * wl.hq * wl.d * 2
    tflops = dense_flops / (ms["target"] * 1e-3) / 1e12
    own = np.minimum(t // wl.r, nblk)
    idx_flops = 3 * int(own.sum()) * 2 * wl.h_i * wl.d_i  # z twice recomputed + dq + dkbar
    del inp, kp
    torch.cuda.empty_cache()
    return {"workload": wl.name, "ms": ms, "total_ms": sum(ms.values()),
            "target_roofline": {"bound": "mfma", "achieved": tflops, "peak": 2500.0,
                                "unit": "TFLOP/s", "frac": tflops / 2500.0,
                                "flops_per_call": dense_flops},
            "indexer_bwd_tflops": idx_flops / (ms["indexer_bwd"] * 1e-3) / 1e12}


def bench_varlen(torch, Q, n_seqs=16, total=131072, floor=2048, reps=3):
    """A packed (THD) prefill batch: n_seqs sequences of a seeded length mix summing to
    `total` tokens (each a whole prompt: its queries are all its tokens), model shapes
    of prefill128k; the whole varlen prefill per call, and its attention alone."""
    import numpy as np
    from synth import generate_varlen, serving_lengths, workload
    wl = workload("prefill128k")
    lens = serving_lengths(n_seqs, total, floor, seed=7)
    inp = generate_varlen(wl, [(n, n) for n in lens], device="cuda")
    max_len = max(lens)
    plan = Q.VarlenPlan(n_seqs, total, max_len, max_len, wl.hq, wl.d, wl.d_i, wl.budget,
                        device="cuda")
    scale = 1.0 / math.sqrt(wl.d)

    def run():
        return Q.qsa_prefill_varlen_forward(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["w"],
                                            inp["k_idx"], inp["cu_q"], inp["cu_k"],
                                            budget=wl.budget, max_lq=max_len, max_lk=max_len,
                                            scale=scale, plan=plan)

    def attn():
        return Q.qsa_sparse_attn_varlen_fwd(inp["q"], inp["k"], inp["v"], plan.sel, inp["cu_q"],
                                            inp["cu_k"], scale=scale, out=plan.out, lse=plan.lse,
                                            max_lk=max_len)

    ms = {}
    for name, f in (("forward", run), ("attention", attn)):
        f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            f()
        b.record()
        torch.cuda.synchronize()
        ms[name] = a.elapsed_time(b) / reps
    t = np.concatenate([np.arange(n, dtype=np.int64) for n in lens])
    a_flops = attention_flops(wl, t)
    del inp, plan
    torch.cuda.empty_cache()
    return {"workload": f"{n_seqs} packed prompts of prefill128k shapes, {total} tokens",
            "lengths": lens, "row_chunk": 16384 // n_seqs, "ms": ms["forward"],
            "tokens_per_s": total / (ms["forward"] * 1e-3), "attention_ms": ms["attention"],
            "attention_roofline": {"bound": "mfma",
                                   "achieved": a_flops / ms["attention"] / 1e9,
                                   "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                                   "frac": a_flops / ms["attention"] / 1e9 / MFMA_BF16_PEAK_TFS,
                                   "algorithmic_flops_per_call": a_flops}}


def bench_pool_encoding(torch, Q, n_tok=1 << 20, d_i=128, rope_dim=64, reps=5):
    """Pooling of 1M raw indexer keys (262144 blocks), plain and with the rotary
    encoding of the pooled keys fused in; HBM roofline on read + write bytes."""
    import torch as _t
    g = _t.Generator(device="cuda").manual_seed(17)
    k = (_t.randn((n_tok, d_i), generator=g, device="cuda") / math.sqrt(d_i)).to(_t.bfloat16)
    out = _t.empty((n_tok // 4, d_i), dtype=_t.bfloat16, device="cuda")
    ms = {}
    for name, pe in (("plain", None), ("encoded", (rope_dim, 1.0e6))):
        Q.qsa_pool_keys(k, out=out, pe=pe)
        _t.cuda.synchronize()
        a, b = _t.cuda.Event(enable_timing=True), _t.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            Q.qsa_pool_keys(k, out=out, pe=pe)
        b.record()
        _t.cuda.synchronize()
        ms[name] = a.elapsed_time(b) / reps
    nbytes = n_tok * d_i * 2 + (n_tok // 4) * d_i * 2
    del k, out
    return {"workload": f"{n_tok} raw indexer keys, d_I {d_i}, r 4; encoding rope_dim "
                        f"{rope_dim}", "plain_us": ms["plain"] * 1e3,
            "encoded_us": ms["encoded"] * 1e3,
            "roofline": {"bound": "hbm", "achieved": nbytes / ms["encoded"] / 1e6,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": nbytes / ms["encoded"] / 1e6 / HBM_PEAK_GBS,
                         "algorithmic_bytes_per_call": nbytes}}


def cpu_baseline(wl, inp, budget_s):
    """The oracle, as it stands, on evenly spread query rows of the same workload."""
    import numpy as np
    import torch

    from oracle import qsa_oracle as O

    def bits(t):
        return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    k_dev, v_dev = inp["k"], inp["v"]

    def fetch(toks):
        tt = torch.from_numpy(toks).to(k_dev.device)
        return O.bf16_to_f64(bits(k_dev[tt])), O.bf16_to_f64(bits(v_dev[tt]))

    qib, kib = bits(inp["q_idx"]), bits(inp["k_idx"])
    w = inp["w"].cpu().numpy()
    prefix = None if inp["k_pooled_prefix"] is None else bits(inp["k_pooled_prefix"])
    t0 = time.perf_counter()
    O.pool_keys(kib, wl.r)
    t_pool = time.perf_counter() - t0
    order = np.random.default_rng(0).permutation(wl.lq)
    done, t_rows = 0, 0.0
    while t_rows < budget_s and done < len(order):
        rows = np.sort(order[done:done + 4])

        class _Q:  # the sampled q rows, addressed by absolute row
            shape = (wl.lq, wl.hq, wl.d)
            data = {int(r): bits(inp["q"][int(r)]) for r in rows}

            def __getitem__(self, i):
                return self.data[int(i)]

        t0 = time.perf_counter()
        O.forward_prefill(_Q(), None, None, qib, w, kib, r=wl.r, budget=wl.budget,
                          q_pos0=wl.q_pos0, k_pooled_prefix_bits=prefix, rows=rows,
                          n_keys=wl.lk, fetch_kv=fetch)
        t_rows += time.perf_counter() - t0 - t_pool  # each call pools again; count it once
        done += len(rows)
    total = t_rows + t_pool * done / wl.lq
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = 1
    cores = len(os.sched_getaffinity(0))
    return {"value": done / total, "unit": "tokens/s", "cores": min(cores, blas),
            "kind": "oracle",
            "sample": f"{done} random query rows of {wl.name} (whole path per row: scores over "
                      f"all earlier blocks, top-k, fp64 attention), pooling amortised per row; "
                      f"{total:.1f} s of CPU time on {cores} cores, BLAS threads {blas}"}


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_sparse_attention_06_amd as Q
    from synth import decode_query_sets, generate, workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return
    if args.tile_only:
        tile_only(torch, Q, args.workload, args.tile_only)
        return

    wl = workload(args.workload)
    inp = generate(wl, device=dev)
    torch.cuda.synchronize()
    progress(f"inputs of {wl.name} resident")
    wall, attn_ms, plan = bench_prefill(args, torch, Q, wl, inp)
    step_events = bench_prefill.step_ms
    path = select_path(Q, wl, args.select)
    progress(f"prefill ({path} selection): {wall / args.steps * 1e3:.2f} ms per step, "
             f"attention {attn_ms:.2f} ms")
    other = "plain" if path == "fused" else "fused"
    o_wall, o_attn, o_plan = bench_prefill(args, torch, Q, wl, inp, fused=other == "fused")
    del o_plan
    torch.cuda.empty_cache()
    other_ms = o_wall / args.steps * 1e3
    progress(f"prefill ({other} selection): {other_ms:.2f} ms per step")
    ms_step = wall / args.steps * 1e3
    t = wl.q_pos0 + np.arange(wl.lq, dtype=np.int64)
    a_bytes = attention_bytes(wl, t)
    a_flops = attention_flops(wl, t)
    s_flops = score_flops(wl, t)
    a_tfs = a_flops / (attn_ms * 1e-3) / 1e12
    n_launch = Q.qsa_sparse_attn_fwd_launches(wl.lq, wl.lk, wl.hkv, wl.d)
    rows_pl = Q.qsa_sparse_attn_fwd_rows_per_launch(wl.hkv, wl.d)
    traffic = counted_traffic()
    score_ms = bench_score_gemm(torch, Q, wl, inp, plan, args.row_chunk)
    progress(f"score GEMM alone: {score_ms:.2f} ms per step")
    s_tfs = s_flops / (score_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": wl.lq * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "seq_len": wl.lk, "query_tokens": wl.lq,
                   "q_pos0": wl.q_pos0, "heads": f"{wl.hq}q/{wl.hkv}kv", "head_dim": wl.d,
                   "indexer": f"{wl.h_i}x{wl.d_i}", "r": wl.r, "budget": wl.budget,
                   "row_chunk": args.row_chunk, "global_batch": 1, "parallelism": "single GPU"},
        # The dominant kernel (the attention) on its MFMA roofline: algorithmic flops
        # (kept tokens x heads x d x 4) over the live HIP-event duration of the call.
        "roofline": {"kernel": "sparse_attn_kernel (kept-token gather + MFMA)", "bound": "mfma",
                     "achieved": a_tfs, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": a_tfs / MFMA_BF16_PEAK_TFS,
                     "traffic": traffic,
                     "traffic_source": ("bytes beyond L2 per call (MALL or HBM), scaled "
                                        "FETCH_SIZE + WRITE_SIZE from rocprofv3 --pmc runs in "
                                        "profiles/sparse_attn_prefill128k_counters.md; null "
                                        "when the attention sources changed since"),
                     "per": f"one qsa_sparse_attn_fwd call over all {wl.lq} rows = "
                            f"{n_launch} launches of up to {rows_pl} (row, KV group) waves",
                     "launches_per_call": n_launch,
                     "algorithmic_flops_per_call": a_flops, "avg_call_ms": attn_ms,
                     "algorithmic_flops_per_launch": a_flops / n_launch,
                     "avg_launch_ms": attn_ms / n_launch},
        "mfma_fractions": {
            "attention": a_tfs / MFMA_BF16_PEAK_TFS,
            "score_gemm": s_tfs / MFMA_BF16_PEAK_TFS,
            "prefill_step": (a_flops + s_flops) / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
            "score_gemm_ms": score_ms, "score_gemm_flops_per_step": s_flops,
            "attention_flops_per_call": a_flops, "peak_TFLOPs": MFMA_BF16_PEAK_TFS},
        "stages_ms": {"select (pool + scores + top-k)": ms_step - attn_ms, "attention": attn_ms},
        "select_path": path,
        "other_select_path": {"path": other, "ms_per_step": other_ms,
                              "select_ms": other_ms - o_attn},
        "step_ms_events": percentiles(step_events),
    }
    kv_mib = (2 * wl.lk * wl.hkv * wl.d * 2) >> 20
    ceil_rand = gather_ceiling(torch, Q, dev, kv_mib, sequential=False)
    ceil_seq = gather_ceiling(torch, Q, dev, 2048, sequential=True)
    ceil_l2 = gather_ceiling(torch, Q, dev, 2, sequential=False)  # L2-resident on every XCD
    progress(f"gather ceiling: {ceil_rand:.0f} GB/s random, {ceil_seq:.0f} GB/s sequential, "
             f"{ceil_l2:.0f} GB/s from L2")
    beyond = traffic / (attn_ms * 1e-3) / 1e9 if traffic else None
    line["gather"] = {
        "algorithmic_bytes_per_call": a_bytes,
        "effective_GBs": a_bytes / (attn_ms * 1e-3) / 1e9,
        "effective_note": "kept K/V rows + q/out/sel/lse per call over its duration; counts "
                          "L2 and MALL hits, so it is no HBM figure and has no fraction",
        "beyond_l2_bytes_per_call": traffic, "beyond_l2_GBs": beyond,
        "random_gather_ceiling_GBs": ceil_rand, "random_buffer_MiB": kv_mib,
        "sequential_stream_GBs": ceil_seq, "sequential_buffer_MiB": 2048,
        "l2_resident_gather_GBs": ceil_l2, "l2_resident_buffer_MiB": 2,
        # time if the L2 hits and the fetches beyond L2 were served one after the other,
        # each at its measured ceiling
        "serial_model_ms": ((a_bytes - traffic) / ceil_l2 + traffic / ceil_rand) / 1e6
        if traffic else None,
        "beyond_l2_frac_of_random_ceiling": beyond / ceil_rand if beyond else None}
    # The score GEMM's output stream against the write ceiling (a chunk-sized buffer).
    w_bytes = score_write_bytes(wl)
    chunk_bytes = min(args.row_chunk, wl.lq) * Q.score_ld(wl.lk // wl.r) * 4
    w_plain = write_ceiling(torch, dev, chunk_bytes, nontemporal=False)
    w_nt = write_ceiling(torch, dev, chunk_bytes, nontemporal=True)
    progress(f"write ceiling: {w_plain:.0f} GB/s plain, {w_nt:.0f} GB/s non-temporal")
    w_best = max(w_plain, w_nt)
    line["score_writes"] = {
        "bytes_per_step": w_bytes, "GBs": w_bytes / (score_ms * 1e-3) / 1e9,
        "write_ceiling_GBs": {"plain": w_plain, "nontemporal": w_nt},
        "ceiling_buffer_MiB": chunk_bytes >> 20,
        "frac_of_write_ceiling": w_bytes / (score_ms * 1e-3) / 1e9 / w_best,
        "floor_ms_at_ceiling": w_bytes / (w_best * 1e9) * 1e3,
        "note": ("the two-kernel selection's score GEMM (score_gemm_ms) stores every fp32 score "
                 "non-temporal; its time cannot fall below the floor. The fused "
                 "selection stores only list entries.")}
    if not args.no_tile and wl.n_sel <= 512:
        line["attention_tile"] = bench_attention_tile(torch, Q, wl, inp, plan.sel)
    if not args.no_backward:
        b_ms = bench_backward(torch, Q, wl, inp, plan)
        b_bytes = backward_bytes(wl, t)
        b_gbs = b_bytes / (b_ms * 1e-3) / 1e9
        progress(f"backward: {b_ms:.1f} ms")
        b_flops = a_flops * 5 // 2  # 5 products over the kept tokens: S, dP, dV, dQ, dK
        b_tfs = b_flops / (b_ms * 1e-3) / 1e12
        line["backward"] = {
            "workload": wl.name, "what": "dq, dk, dv of the sparse attention (fp32) from out, "
            "lse and a random bf16 dout; inverse selection included",
            "ms": b_ms, "tokens_per_s": wl.lq / (b_ms * 1e-3),
            "roofline": {"bound": "mfma", "achieved": b_tfs, "peak": MFMA_BF16_PEAK_TFS,
                         "unit": "TFLOP/s", "frac": b_tfs / MFMA_BF16_PEAK_TFS,
                         "algorithmic_flops_per_call": b_flops},
            "moved_bytes_GBs": b_gbs, "moved_bytes_per_call": b_bytes,
            "moved_bytes_note": "the design's own traffic (K/V rows, each (block, row) pair's "
                                "q and dout, gradients), not algorithmic bytes; no fraction"}
    del inp, plan
    torch.cuda.empty_cache()
    if not args.no_warmup:
        line["indexer_warmup"] = bench_warmup(torch, Q)
        progress("indexer warm-up done")
    line["pool_encoding"] = bench_pool_encoding(torch, Q)
    progress(f"pooling: {line['pool_encoding']['plain_us']:.1f} us plain, "
             f"{line['pool_encoding']['encoded_us']:.1f} us encoded")
    if not args.no_varlen:
        line["varlen"] = bench_varlen(torch, Q)
        progress(f"varlen: {line['varlen']['ms']:.2f} ms per packed batch")
    if not args.no_decode:
        dwl = workload("decode1m")
        dinp = generate(dwl, device=dev)
        qsets = decode_query_sets(dwl, 16, device=dev)
        torch.cuda.synchronize()
        s_dec = bench_decode(args, torch, Q, dwl, dinp, query_sets=qsets)
        s_dec_same = bench_decode(args, torch, Q, dwl, dinp)
        progress(f"decode: {s_dec * 1e6:.1f} us per step")
        # The MTP layer reuses the main layer's selection: its step is the decode
        # attention alone (its own cache; the same bytes are read here).
        mtp_plan = Q.DecodePlan(dwl.batch, dwl.hq, dwl.d, dwl.lk, dwl.budget, device=dev)
        mtp_sels = []
        for x in qsets:
            Q.qsa_decode_forward(x["q"], x["q_idx"], x["w"], dinp["k_pooled"],
                                 dinp["k_cache"], dinp["v_cache"], dinp["seq_lens"],
                                 budget=dwl.budget, plan=mtp_plan)
            mtp_sels.append(mtp_plan.sel.clone())
        mtp_i = [0]

        def mtp_call():
            i = mtp_i[0] % len(qsets)
            mtp_i[0] += 1
            Q.qsa_sparse_attn_decode(qsets[i]["q"], dinp["k_cache"], dinp["v_cache"],
                                     dinp["seq_lens"], mtp_sels[i])

        mtp_s = time_calls(torch, mtp_call, 32)
        progress(f"MTP decode attention over the reused selection: {mtp_s * 1e6:.1f} us")
        own = (dwl.lk - 1) // dwl.r
        d_bytes = dwl.batch * (own * dwl.d_i * 2 + dwl.budget * dwl.hkv * 2 * dwl.d * 2 +
                               dwl.hq * dwl.d * 2 * 2)
        line["mtp_reuse"] = {
            "what": "MTP layer attending over the main layer's selections (no indexer)",
            "prefill128k_ms": attn_ms, "prefill128k_main_step_ms": ms_step,
            "decode1m_us": mtp_s * 1e6, "decode1m_main_step_us": s_dec * 1e6}
        line["decode"] = {"workload": dwl.name, "batch": dwl.batch, "context": dwl.lk,
                          "value": dwl.batch / s_dec, "unit": "tokens/s", "ms_per_step": s_dec * 1e3,
                          "steps": args.decode_steps,
                          "queries": "16 seeded query sets in turn (each step selects and "
                                     "gathers other blocks of the same caches)",
                          "ms_per_step_same_query": s_dec_same * 1e3,
                          "roofline": {"bound": "hbm", "achieved": d_bytes / s_dec / 1e9,
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": d_bytes / s_dec / 1e9 / HBM_PEAK_GBS,
                                       "algorithmic_bytes_per_step": d_bytes}}
        if not args.no_paged:
            P = 64
            kp, vp, table = paged_copy(torch, dinp["k_cache"], dinp["v_cache"], P)
            del dinp["k_cache"], dinp["v_cache"]
            torch.cuda.empty_cache()
            s_pg = bench_decode(args, torch, Q, dwl, dinp, paged=(kp, vp, table, P),
                                query_sets=qsets)
            progress(f"paged decode: {s_pg * 1e6:.1f} us per step")
            line["decode_paged"] = {
                "workload": f"{dwl.name}, K/V in shuffled pages of {P} tokens",
                "page_size": P, "value": dwl.batch / s_pg, "unit": "tokens/s",
                "ms_per_step": s_pg * 1e3,
                "roofline": {"bound": "hbm", "achieved": d_bytes / s_pg / 1e9,
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": d_bytes / s_pg / 1e9 / HBM_PEAK_GBS,
                             "algorithmic_bytes_per_step": d_bytes}}
            del kp, vp, table
        del dinp
        torch.cuda.empty_cache()
    if not args.no_other and wl.name == "prefill128k":
        line["other_prefill"] = {n: bench_other_prefill(torch, Q, n, args.select)
                                 for n in ("prefill32k", "chunked1m")}
        progress("other prefill workloads: " + ", ".join(
            f"{n} {v['ms_per_step']:.2f} ms" for n, v in line["other_prefill"].items()))
    if not args.no_cpu_baseline:
        inp = generate(wl, device=dev)
        line["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
        progress("cpu baseline done")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
