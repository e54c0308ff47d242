"""The multi-row attention tile (qsa_sparse_attn_fwd_tiled) against the oracle.

Each row's output and log-sum-exp are checked against the oracle's attention over that
row's kept tokens (the same bar as the per-row kernel), on random selections (rows
share few blocks) and on selections where neighbouring rows share most of their blocks
(the union path's case), with the union forced (min_shared 0), chosen by the sampled
overlap (32) and never taken (65); partial last tiles, model shapes and the 128K
workload in the launch configuration of a full call."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_06_amd as Q
from oracle import qsa_oracle as O
from parity import LSE_ABS, bits, compare_output
from synth import generate, workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


def _randn_bf16(shape, seed, scale=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(torch.bfloat16)


def _selection(pos, n_sel, seed, shared):
    """Valid selections (ascending, own block last, -1 padded). shared=False: each row
    draws its blocks independently; shared=True: the 4 rows of a tile draw from one
    random order of the first row's candidates, row j taking a window shifted by j/8
    of its length, so neighbours share about 7/8 of their blocks."""
    rng = np.random.default_rng(seed)
    sel = np.full((len(pos), n_sel), -1, dtype=np.int32)
    perm = None
    for i, t in enumerate(pos):
        own = int(t) // 4
        if shared and i % 4 == 0:
            perm = rng.permutation(own)
        if shared:
            cand = perm[perm < own]
            m = min(n_sel - 1, len(cand))
            shift = (i % 4) * max(m // 8, 1)
            pick = np.roll(cand, -shift)[:m] if m else np.zeros(0, int)
        else:
            m = min(n_sel - 1, own)
            pick = rng.choice(own, size=m, replace=False) if m else np.zeros(0, int)
        sel[i, :m] = np.sort(pick)
        sel[i, m] = own
    return sel


def _check_rows(q, k, v, sel_np, pos, rows, out, lse, where):
    d = q.shape[2]
    lk = k.shape[0]
    qb, kb, vb = bits(q), bits(k), bits(v)
    ref = np.zeros((len(rows), q.shape[1], d))
    ref_lse = np.zeros((len(rows), q.shape[1]))
    for j, i in enumerate(rows):
        toks = O.kept_tokens(sel_np[i], int(pos[i]), 4, lk)
        ref[j], ref_lse[j] = O.attend(O.bf16_to_f64(qb[i]), O.bf16_to_f64(kb[toks]),
                                      O.bf16_to_f64(vb[toks]), 1 / math.sqrt(d))
    max_abs, rel = compare_output(out[torch.from_numpy(np.asarray(rows)).to(DEV)], ref, where)
    got_lse = lse.double().cpu().numpy()[rows]
    lse_err = float(np.max(np.abs(got_lse - ref_lse)))
    assert lse_err <= LSE_ABS, f"{where}: lse {lse_err:.3e}"
    _say(f"  {where}: max-abs {max_abs:.2e} rel-L2 {rel:.2e} lse {lse_err:.2e}")


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("min_shared", [0, 32, 65])
@pytest.mark.parametrize("lq,lk,q_pos0,hq,hkv,d,budget", [
    (701, 4102, 3401, 24, 2, 256, 2048),   # model shape, ragged Lk, partial last tile
    (513, 513, 0, 16, 1, 256, 64),         # 16 heads per group, rows with few blocks
    (302, 1200, 898, 2, 2, 128, 16),       # 1 head per group, d = 128
    (1024, 1024, 0, 8, 2, 128, 256),       # whole-row selections at the start
])
def test_tiled_attention_against_oracle(lq, lk, q_pos0, hq, hkv, d, budget, min_shared, shared):
    _say(f"tiled attn lq={lq} lk={lk} q_pos0={q_pos0} hq={hq}/{hkv} d={d} K={budget} "
         f"min_shared={min_shared} shared={shared}")
    seed = lq + 3 * min_shared + (7 if shared else 0)
    sc = 1 / math.sqrt(d)
    q = _randn_bf16((lq, hq, d), seed, sc)
    k = _randn_bf16((lk, hkv, d), seed + 1, sc)
    v = _randn_bf16((lk, hkv, d), seed + 2, sc)
    pos = q_pos0 + np.arange(lq)
    sel_np = _selection(pos, budget // 4, seed, shared)
    sel = torch.from_numpy(sel_np).to(DEV)
    out, lse = Q.qsa_sparse_attn_fwd_tiled(q, k, v, sel, q_pos0=q_pos0, min_shared=min_shared)
    torch.cuda.synchronize()
    _check_rows(q, k, v, sel_np, pos, np.arange(lq), out, lse, f"tiled lq={lq} d={d}")
    # and against the per-row kernel on the same selections (fp32 summation order only)
    ref_out, _ = Q.qsa_sparse_attn_fwd(q, k, v, sel, q_pos0=q_pos0)
    diff = (out.float() - ref_out.float()).abs().max().item()
    assert diff <= 2e-2, f"tiled vs per-row kernel: {diff:.3e}"


def test_tiled_attention_identical_rows_match_per_row_kernel():
    # When the 4 rows of every tile keep the very same blocks, the union is each row's
    # own list and no column is masked: the steps are those of the per-row kernel, so
    # the outputs are bit-identical.
    _say("tiled attn, identical selections within each tile")
    lq, lk, hq, hkv, d = 512, 8192, 24, 2, 256
    q_pos0 = lk - lq
    q = _randn_bf16((lq, hq, d), 5, 1 / math.sqrt(d))
    k = _randn_bf16((lk, hkv, d), 6, 1 / math.sqrt(d))
    v = _randn_bf16((lk, hkv, d), 7, 1 / math.sqrt(d))
    rng = np.random.default_rng(11)
    n_sel = 512
    sel_np = np.full((lq, n_sel), -1, dtype=np.int32)
    for tile in range(lq // 4):
        t0 = q_pos0 + 4 * tile  # the tile's rows share block t0 // 4 unless they cross one
        own = t0 // 4
        pick = np.sort(rng.choice(own, size=n_sel - 1, replace=False))
        for j in range(4):
            sel_np[4 * tile + j, :n_sel - 1] = pick
            sel_np[4 * tile + j, n_sel - 1] = own  # q_pos0 % 4 == 0: the 4 rows share it
    sel = torch.from_numpy(sel_np).to(DEV)
    out_t, lse_t = Q.qsa_sparse_attn_fwd_tiled(q, k, v, sel, q_pos0=q_pos0, min_shared=0)
    out_r, lse_r = Q.qsa_sparse_attn_fwd(q, k, v, sel, q_pos0=q_pos0)
    torch.cuda.synchronize()
    assert torch.equal(out_t, out_r)
    # the log-sum-exp's last two operations (ln of the sum, plus the max) are compiled
    # separately in the two kernels and may round differently: a few ulps
    lse_ulps = ((lse_t - lse_r).abs() / torch.finfo(torch.float32).eps / lse_r.abs()).max().item()
    assert lse_ulps <= 4, f"lse differs by {lse_ulps:.1f} ulps"


@pytest.mark.parametrize("min_shared", [0, 32])
def test_tiled_attention_128k_sampled(min_shared):
    # The 128K workload's own selections (the library's selection path), the whole call
    # in its launch configuration; rows at tile and launch edges and random rows
    # against the oracle.
    wl = workload("prefill128k")
    _say(f"tiled attn 128K min_shared={min_shared}")
    inp = generate(wl, device=DEV)
    sel, _ = Q.qsa_prefill_select(inp["q_idx"], inp["w"], inp["k_idx"], lk=wl.lk,
                                  budget=wl.budget, q_pos0=wl.q_pos0,
                                  k_pooled_prefix=inp["k_pooled_prefix"], row_chunk=16384)
    out, lse = Q.qsa_sparse_attn_fwd_tiled(inp["q"], inp["k"], inp["v"], sel, q_pos0=wl.q_pos0,
                                           min_shared=min_shared)
    torch.cuda.synchronize()
    gen = Q.qsa_sparse_attn_fwd_rows_per_launch(wl.hkv, wl.d)
    rng = np.random.default_rng(min_shared + 1)
    rows = np.unique(np.concatenate([[0, 1, 2, 3, 4, 5, 2045, 2046, 2047, 2048, wl.lq - 1],
                                     rng.integers(0, wl.lq, 40)]))
    rows = rows[rows < wl.lq]
    sel_np = sel.cpu().numpy()
    pos = wl.q_pos0 + np.arange(wl.lq)
    _check_rows(inp["q"], inp["k"], inp["v"], sel_np, pos, rows, out, lse,
                f"tiled 128K (launch rows {gen})")
