"""Index reuse by the multi-token-prediction module on an MI355X: the MTP layer runs no
indexer and attends over the selections of the main model's layer at the same
positions ([DR]: the MTP module reuses the top-k indices). Its attention, through the
C ABI, against the oracle on those reused selections, for prefill and decode."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_06_amd as Q
from oracle import qsa_oracle as O
from parity import bits, compare_output, LSE_ABS
from synth import generate, workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _randn_bf16(shape, seed, scale):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(torch.bfloat16)


def test_mtp_prefill_reuses_main_selection():
    wl = workload("prefill32k", lq=6000, lk=6000, seed=31)
    inp = generate(wl, device=DEV)
    _, _, sel, _ = Q.qsa_prefill_forward(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["w"],
                                         inp["k_idx"], budget=wl.budget)
    sd = 1 / math.sqrt(wl.d)
    q2 = _randn_bf16(inp["q"].shape, 1, sd)
    k2 = _randn_bf16(inp["k"].shape, 2, sd)
    v2 = _randn_bf16(inp["v"].shape, 3, sd)
    out2, lse2 = Q.qsa_sparse_attn_fwd(q2, k2, v2, sel)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 5999], np.random.default_rng(5).integers(0, 6000, 40)]))
    sel_np = sel.cpu().numpy()
    qf, kf, vf = (O.bf16_to_f64(bits(t)) for t in (q2, k2, v2))
    ref = np.zeros((len(rows), wl.hq, wl.d))
    for j, i in enumerate(rows):
        toks = O.kept_tokens(sel_np[i], int(i), 4, wl.lk)
        ref[j], ref_lse = O.attend(qf[i], kf[toks], vf[toks], sd)
        assert np.abs(lse2[i].double().cpu().numpy() - ref_lse).max() <= LSE_ABS
    compare_output(out2[torch.from_numpy(rows).to(DEV)], ref, "MTP prefill")


def test_mtp_decode_reuses_main_selection():
    seq = [65536, 30001, 777, 2048]
    wl = workload("decode1m", batch=len(seq), lk=65536)
    inp = generate(wl, device=DEV, seq_lens=seq)
    _, _, sel = Q.qsa_decode_forward(inp["q"], inp["q_idx"], inp["w"], inp["k_pooled"],
                                     inp["k_cache"], inp["v_cache"], inp["seq_lens"],
                                     budget=wl.budget)
    sd = 1 / math.sqrt(wl.d)
    q2 = _randn_bf16(inp["q"].shape, 4, sd)
    k2 = _randn_bf16(inp["k_cache"].shape, 5, sd)  # the MTP layer's own cache
    v2 = _randn_bf16(inp["v_cache"].shape, 6, sd)
    out2, lse2 = Q.qsa_sparse_attn_decode(q2, k2, v2, inp["seq_lens"], sel)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    for b, n in enumerate(seq):
        toks = O.kept_tokens(sel_np[b], n - 1, 4, n)
        tt = torch.from_numpy(toks).to(DEV)
        ref, ref_lse = O.attend(O.bf16_to_f64(bits(q2[b])), O.bf16_to_f64(bits(k2[b][tt])),
                                O.bf16_to_f64(bits(v2[b][tt])), sd)
        compare_output(out2[b], ref, f"MTP decode b={b}")
        assert np.abs(lse2[b].double().cpu().numpy() - ref_lse).max() <= LSE_ABS
