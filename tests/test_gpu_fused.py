"""The fused score/top-k selection (qsa_prefill_select_fused) against the two-kernel
selection and the oracle. Both score blocks with the same fp32 arithmetic and select
exactly with the same tie rule, so the kept ids must be identical on every row; rows
whose list comes out short or overflows (forced here with extreme tunings) go through
the exact fallback and must still match."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_06_amd as Q
from oracle import qsa_oracle as O
from parity import bits, check_selection_row, compare_output, score_abs_tol
from synth import generate, workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


def _both(wl, inp, row_chunk, tuning=None):
    args = (inp["q_idx"], inp["w"], inp["k_idx"])
    kw = dict(lk=wl.lk, budget=wl.budget, q_pos0=wl.q_pos0, k_pooled_prefix=inp["k_pooled_prefix"],
              row_chunk=row_chunk)
    ref, kp_ref = Q.qsa_prefill_select(*args, fused=False, **kw)
    ref, kp_ref = ref.clone(), kp_ref.clone()
    got, kp = Q.qsa_prefill_select(*args, fused=True, tuning=tuning, **kw)
    torch.cuda.synchronize()
    assert torch.equal(kp, kp_ref)
    return got, ref


@pytest.mark.parametrize("name,row_chunk,over", [
    ("tiny", 4096, {}),
    ("tiny", 300, dict(lq=1001, lk=1001)),                       # ragged chunks and tiles
    ("prefill32k", 16384, {}),
    ("prefill32k", 2500, dict(lq=12000, lk=40000, q_pos0=28000, pooled_prefix_blocks=5000)),
    ("prefill32k", 16384, dict(smooth=100)),                      # correlated rows
    ("prefill128k", 16384, {}),
    ("prefill128k", 65536, {}),                                   # the bench's chunks: 1024 tiles, one piece
    ("chunked1m", 8192, {}),                                      # 262K candidates a row
    ("prefill32k", 32768, {}),                                    # one key-range piece
    ("prefill32k", 9000, {}),                                     # three pieces
    # rows whose candidates cross the 65536-block window of the list select's bitmap
    ("prefill32k", 1000, dict(lq=1000, lk=263000, q_pos0=262000, pooled_prefix_blocks=65500)),
])
def test_fused_selection_equals_two_kernel_selection(name, row_chunk, over):
    wl = workload(name, **over)
    _say(f"fused vs two-kernel {wl.name} lq={wl.lq} lk={wl.lk} q_pos0={wl.q_pos0} "
         f"chunk={row_chunk} {over}")
    inp = generate(wl, device=DEV)
    got, ref = _both(wl, inp, row_chunk)
    bad = (got != ref).any(dim=1).nonzero().flatten()
    assert bad.numel() == 0, f"{bad.numel()} rows differ, first {bad[:5].tolist()}"


@pytest.mark.parametrize("tuning,what", [
    ((1, 1, 0), "threshold at the best sample: short lists, most rows fall back"),
    ((0, 0, 64), "capacity below m: every long row overflows and falls back"),
    ((300, 3, 0), "a noisy threshold: a mix of listed and fallback rows"),
])
def test_fused_fallback_rows(tuning, what):
    wl = workload("prefill32k", lq=6000, lk=40000, q_pos0=34000, pooled_prefix_blocks=5000)
    _say(f"fused fallback {tuning}: {what}")
    inp = generate(wl, device=DEV)
    got, ref = _both(wl, inp, 2500, tuning=tuning)
    bad = (got != ref).any(dim=1).nonzero().flatten()
    assert bad.numel() == 0, f"{bad.numel()} rows differ, first {bad[:5].tolist()}"


def test_fused_selection_against_oracle():
    # Rows of the chunked 1M workload (selection chunks of 8192 rows), the oracle's own
    # end-to-end selection, and the attention over the fused path's selection.
    wl = workload("chunked1m")
    inp = generate(wl, device=DEV)
    plan = Q.PrefillPlan(wl.lq, wl.lk, wl.hq, wl.hkv, wl.d, wl.h_i, wl.d_i, wl.budget,
                         row_chunk=8192, device=DEV, fused=True)
    sel, kp = Q.qsa_prefill_select(inp["q_idx"], inp["w"], inp["k_idx"], lk=wl.lk,
                                   budget=wl.budget, q_pos0=wl.q_pos0,
                                   k_pooled_prefix=inp["k_pooled_prefix"], plan=plan)
    out, lse = Q.qsa_sparse_attn_fwd(inp["q"], inp["k"], inp["v"], sel, q_pos0=wl.q_pos0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([rng.choice(wl.lq, 96, replace=False),
                                     inp["aligned_rows"][:32], [0, wl.lq - 1]])).astype(np.int64)
    _say(f"fused vs oracle chunked1m rows={len(rows)}")
    rows_t = torch.from_numpy(rows).to(DEV)
    qib, w_np = bits(inp["q_idx"]), inp["w"].cpu().numpy()
    kpb = bits(kp)
    kp64 = O.bf16_to_f64(kpb)
    own = (wl.q_pos0 + rows) // wl.r
    sc = O.index_scores(O.bf16_to_f64(qib[rows]), w_np[rows], kp64, wl.q_pos0 + rows, wl.r)
    tol = score_abs_tol(O.bf16_to_f64(qib[rows]), w_np[rows], kp64, own)
    sel_np = sel[rows_t].cpu().numpy()
    n_exact = sum(check_selection_row(sel_np[j], sc[j, :own[j]], int(own[j]), wl.n_sel,
                                      f"fused row {i}", abs_tol=tol[j])
                  for j, i in enumerate(rows))
    assert n_exact >= len(rows) - 1
    ref = np.zeros((len(rows), wl.hq, wl.d))
    for j, i in enumerate(rows):
        toks = O.kept_tokens(sel_np[j], wl.q_pos0 + int(i), wl.r, wl.lk)
        tt = torch.from_numpy(toks).to(DEV)
        ref[j], _ = O.attend(O.bf16_to_f64(bits(inp["q"][int(i)])),
                             O.bf16_to_f64(bits(inp["k"][tt])), O.bf16_to_f64(bits(inp["v"][tt])),
                             1 / math.sqrt(wl.d))
    max_abs, rel = compare_output(out[rows_t], ref, "fused chunked1m")
    _say(f"  exact_sel={n_exact}/{len(rows)} max_abs={max_abs:.2e} rel_l2={rel:.2e}")
