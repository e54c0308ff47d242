"""Packed variable-length (THD) prefill on an MI355X, through the C ABI: against the
oracle on sampled rows of every sequence, and bit for bit against one-sequence calls."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_06_amd as Q
from oracle import qsa_oracle as O
from parity import bits, check_selection_row, compare_output, score_abs_tol, LSE_ABS
from synth import generate_varlen, workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


def _model_wl(budget=2048, seed=11):
    return workload("prefill32k", budget=budget, seed=seed, needle_spacing=1024)


def _run(inp, wl, **kw):
    return Q.qsa_prefill_varlen_forward(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["w"],
                                        inp["k_idx"], inp["cu_q"], inp["cu_k"],
                                        budget=wl.budget, **kw)


def _check_against_oracle(inp, wl, out, lse, sel, kp, rows):
    cq, ck = inp["cu_q"].cpu().numpy(), inp["cu_k"].cpu().numpy()
    # Pooled keys: each sequence's complete blocks in its slot, bit-exact.
    kb = bits(inp["k_idx"])
    for b, (lq, lk) in enumerate(inp["lens"]):
        nb = lk // wl.r
        np.testing.assert_array_equal(bits(kp[b, :nb]), O.pool_keys(kb[ck[b]:ck[b + 1]], wl.r))
    res = O.forward_prefill_varlen(bits(inp["q"]), bits(inp["k"]), bits(inp["v"]),
                                   bits(inp["q_idx"]), inp["w"].cpu().numpy(), kb, cq, ck,
                                   r=wl.r, budget=wl.budget, rows=rows)
    sel_np = sel.cpu().numpy()
    seq_of = np.searchsorted(cq, rows, side="right") - 1
    n_exact = 0
    ref = np.zeros((len(rows), wl.hq, wl.d))
    kf, vf = O.bf16_to_f64(bits(inp["k"])), O.bf16_to_f64(bits(inp["v"]))
    qf = O.bf16_to_f64(bits(inp["q"]))
    for j, i in enumerate(rows):
        b = seq_of[j]
        lq, lk = inp["lens"][b]
        t = lk - lq + (i - cq[b])
        tol = score_abs_tol(O.bf16_to_f64(bits(inp["q_idx"][i]))[None],
                            inp["w"][i].double().cpu().numpy()[None],
                            O.bf16_to_f64(res["pooled"][b]), [t // wl.r])[0]
        n_exact += check_selection_row(sel_np[i], res["scores"][j], t // wl.r, wl.n_sel,
                                       f"seq {b} row {i}", abs_tol=tol)
        toks = O.kept_tokens(sel_np[i], t, wl.r, lk) + ck[b]
        ref[j], ref_lse = O.attend(qf[i], kf[toks], vf[toks], 1 / math.sqrt(wl.d))
        assert np.abs(lse[i].cpu().numpy() - ref_lse).max() <= LSE_ABS
    for i, blk in zip(inp["aligned_rows"], inp["aligned_blocks"]):
        assert blk in sel_np[i], f"row {i} lost needle block {blk}"
    rows_t = torch.from_numpy(np.asarray(rows)).to(DEV)
    max_abs, rel = compare_output(out[rows_t], ref, "varlen")
    _say(f"  rows={len(rows)} exact_sel={n_exact} max_abs={max_abs:.2e} rel_l2={rel:.2e}")
    return n_exact


def _sample_rows(inp, n_per_seq, seed):
    rng = np.random.default_rng(seed)
    cq = inp["cu_q"].cpu().numpy()
    rows = []
    for b in range(len(cq) - 1):
        q0, q1 = int(cq[b]), int(cq[b + 1])
        if q1 > q0:
            rows += [q0, q1 - 1] + list(rng.integers(q0, q1, size=min(n_per_seq, q1 - q0)))
    rows += list(inp["aligned_rows"][:32])
    return np.unique(np.asarray(rows, dtype=np.int64))


def test_varlen_model_shapes_against_oracle():
    # Mixed lengths: plain prefills, a chunk after a packed-in prefix, a sequence with
    # no query, one shorter than a block, one longer than the budget many times over.
    lens = [(3000, 3000), (517, 517), (1000, 4093), (0, 12), (5, 5), (2, 3), (6000, 6000)]
    wl = _model_wl()
    _say(f"varlen lens={lens}")
    inp = generate_varlen(wl, lens, device=DEV)
    out, lse, sel, kp = _run(inp, wl, max_lq=6000, max_lk=6000, row_chunk=1024)
    torch.cuda.synchronize()
    rows = _sample_rows(inp, 12, 1)
    n_exact = _check_against_oracle(inp, wl, out, lse, sel, kp, rows)
    assert n_exact >= len(rows) - 2


def test_varlen_many_short_sequences_small_chunks():
    # 24 short sequences (lengths 1..300, some with packed prefixes), chunks of 64 rows.
    rng = np.random.default_rng(5)
    lens = []
    for _ in range(24):
        lk = int(rng.integers(1, 301))
        lens.append((int(rng.integers(1, lk + 1)), lk))
    wl = _model_wl(budget=256)
    _say(f"varlen short lens={lens}")
    inp = generate_varlen(wl, lens, device=DEV)
    out, lse, sel, kp = _run(inp, wl, row_chunk=64)
    torch.cuda.synchronize()
    rows = np.arange(int(inp["cu_q"][-1]))
    n_exact = _check_against_oracle(inp, wl, out, lse, sel, kp, rows)
    assert n_exact >= len(rows) - 2


def test_varlen_equals_one_sequence_calls():
    # Every row's selection and attention depend on its own sequence only: the packed
    # call writes what separate one-sequence calls write, bit for bit.
    lens = [(2048, 2048), (700, 2900), (1500, 1500), (64, 64)]
    wl = _model_wl(seed=12)
    inp = generate_varlen(wl, lens, device=DEV)
    out, lse, sel, kp = _run(inp, wl, row_chunk=512)
    cq, ck = inp["cu_q"].cpu().numpy(), inp["cu_k"].cpu().numpy()
    for b, (lq, lk) in enumerate(lens):
        qs, ks = slice(int(cq[b]), int(cq[b + 1])), slice(int(ck[b]), int(ck[b + 1]))
        o1, l1, s1, k1 = Q.qsa_prefill_forward(inp["q"][qs], inp["k"][ks], inp["v"][ks],
                                               inp["q_idx"][qs], inp["w"][qs], inp["k_idx"][ks],
                                               budget=wl.budget, q_pos0=lk - lq, row_chunk=777)
        torch.cuda.synchronize()
        assert torch.equal(s1, sel[qs]), f"sequence {b}: selection differs"
        assert torch.equal(o1, out[qs]) and torch.equal(l1, lse[qs]), f"sequence {b}: output"
        assert torch.equal(k1, kp[b, : lk // 4]), f"sequence {b}: pooled keys"
