"""Positional encoding of the pooled keys on an MI355X, through the C ABI: the fused
pool + rotary encoding bit for bit against the oracle, and the prefill paths that use
it (one sequence, a chunk after an encoded prefix, packed sequences)."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_06_amd as Q
from oracle import qsa_oracle as O
from parity import bits, check_selection_row, compare_output, score_abs_tol
from synth import generate, generate_varlen, workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("n_tok,d_i,rope_dim,first_block",
                         [(4 * 5000 + 1, 128, 64, 0), (4 * 777, 128, 128, 12345),
                          (4 * 100 + 2, 64, 16, 3), (4 * 262144, 128, 64, 0)])
def test_pool_with_encoding_bit_exact(n_tok, d_i, rope_dim, first_block):
    g = torch.Generator(device=DEV).manual_seed(n_tok)
    k = (torch.randn((n_tok, d_i), generator=g, device=DEV) / math.sqrt(d_i)).to(torch.bfloat16)
    pe = (rope_dim, 1.0e6)
    got = Q.qsa_pool_keys(k, pe=pe, first_block=first_block)
    torch.cuda.synchronize()
    ref = O.pool_keys(bits(k), 4, (rope_dim, float(np.float32(1.0e6))), first_block=first_block)
    np.testing.assert_array_equal(bits(got), ref)


@pytest.mark.parametrize("n_tok,d_i,rope_dim,first_block",
                         [(4 * 3001, 256, 48, 77), (4 * 999 + 1, 512, 512, 5),
                          (4 * 300, 64, 64, 0), (4 * 500, 96, 32, 9), (4 * 123, 1024, 80, 1)])
def test_pool_with_encoding_other_shapes(n_tok, d_i, rope_dim, first_block):
    # partner columns rope_dim/2 apart that are not a power of two (48, 80), a whole-row
    # rotation, and widths taking the per-thread form (96, 1024)
    _say(f"encoded pool n_tok={n_tok} d_i={d_i} rope_dim={rope_dim}")
    g = torch.Generator(device=DEV).manual_seed(n_tok + d_i)
    k = (torch.randn((n_tok, d_i), generator=g, device=DEV) / math.sqrt(d_i)).to(torch.bfloat16)
    got = Q.qsa_pool_keys(k, pe=(rope_dim, 1.0e4), first_block=first_block)
    torch.cuda.synchronize()
    ref = O.pool_keys(bits(k), 4, (rope_dim, 1.0e4), first_block=first_block)
    np.testing.assert_array_equal(bits(got), ref)


def _check_rows(inp, wl, out, sel, kp, rows, pe, q_pos0, prefix_bits=None):
    res = O.forward_prefill(bits(inp["q"]), bits(inp["k"]), bits(inp["v"]), bits(inp["q_idx"]),
                            inp["w"].cpu().numpy(), bits(inp["k_idx"]), r=4, budget=wl.budget,
                            q_pos0=q_pos0, rows=rows, k_pooled_prefix_bits=prefix_bits, pe=pe)
    n_prefix = 0 if prefix_bits is None else len(prefix_bits)
    np.testing.assert_array_equal(bits(kp[n_prefix:]), res["pooled"])
    sel_np = sel.cpu().numpy()
    kp_all = O.bf16_to_f64(res["pooled"] if prefix_bits is None
                           else np.concatenate([prefix_bits, res["pooled"]]))
    rr = np.asarray(rows)
    tol = score_abs_tol(O.bf16_to_f64(bits(inp["q_idx"]))[rr], inp["w"].cpu().numpy()[rr],
                        kp_all, (q_pos0 + rr) // 4)
    n_exact = 0
    for j, i in enumerate(rows):
        n_exact += check_selection_row(sel_np[i], res["scores"][j], (q_pos0 + i) // 4, wl.n_sel,
                                       f"row {i}", abs_tol=tol[j])
    ref = np.zeros((len(rows), wl.hq, wl.d))
    kf, vf = O.bf16_to_f64(bits(inp["k"])), O.bf16_to_f64(bits(inp["v"]))
    qf = O.bf16_to_f64(bits(inp["q"]))
    for j, i in enumerate(rows):
        toks = O.kept_tokens(sel_np[i], q_pos0 + int(i), 4, kf.shape[0])
        ref[j], _ = O.attend(qf[i], kf[toks], vf[toks], 1 / math.sqrt(wl.d))
    compare_output(out[torch.from_numpy(np.asarray(rows)).to(DEV)], ref, "encoded prefill")
    return n_exact


def test_encoded_prefill_against_oracle():
    wl = workload("prefill32k", lq=4096, lk=12288, q_pos0=8192, needle_spacing=0, seed=21)
    inp = generate(wl, device=DEV)
    pe = (64, 1.0e6)
    out, lse, sel, kp = Q.qsa_prefill_forward(inp["q"], inp["k"], inp["v"], inp["q_idx"],
                                              inp["w"], inp["k_idx"], budget=wl.budget,
                                              q_pos0=wl.q_pos0, pe=pe)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 4095], np.random.default_rng(2).integers(0, 4096, 30)]))
    n_exact = _check_rows(inp, wl, out, sel, kp, rows, pe, wl.q_pos0)
    assert n_exact >= len(rows) - 2


def test_encoded_chunk_after_encoded_prefix():
    # The prefix's pooled keys arrive encoded (at their own positions); the chunk's new
    # blocks are encoded from the prefix's end on.
    wl = workload("prefill32k", lq=2048, lk=10240, q_pos0=8192, pooled_prefix_blocks=2048,
                  needle_spacing=0, seed=22)
    inp = generate(wl, device=DEV)
    pe = (128, 1.0e4)
    g = torch.Generator(device=DEV).manual_seed(3)
    raw_prefix = (torch.randn((8192, wl.d_i), generator=g, device=DEV) / math.sqrt(wl.d_i))
    raw_prefix = raw_prefix.to(torch.bfloat16)
    prefix = Q.qsa_pool_keys(raw_prefix, pe=pe)
    out, lse, sel, kp = Q.qsa_prefill_forward(inp["q"], inp["k"], inp["v"], inp["q_idx"],
                                              inp["w"], inp["k_idx"], budget=wl.budget,
                                              q_pos0=wl.q_pos0, k_pooled_prefix=prefix, pe=pe)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 2047], np.random.default_rng(4).integers(0, 2048, 24)]))
    n_exact = _check_rows(inp, wl, out, sel, kp, rows, pe, wl.q_pos0, prefix_bits=bits(prefix))
    assert n_exact >= len(rows) - 2


def test_encoded_varlen_equals_one_sequence_calls():
    lens = [(1500, 1500), (600, 3000), (2048, 2048)]
    wl = workload("prefill32k", seed=23, needle_spacing=0)
    inp = generate_varlen(wl, lens, device=DEV)
    pe = (64, 1.0e6)
    out, lse, sel, kp = Q.qsa_prefill_varlen_forward(inp["q"], inp["k"], inp["v"], inp["q_idx"],
                                                     inp["w"], inp["k_idx"], inp["cu_q"],
                                                     inp["cu_k"], budget=wl.budget, pe=pe)
    cq, ck = inp["cu_q"].cpu().numpy(), inp["cu_k"].cpu().numpy()
    for b, (lq, lk) in enumerate(lens):
        qs, ks = slice(int(cq[b]), int(cq[b + 1])), slice(int(ck[b]), int(ck[b + 1]))
        o1, l1, s1, k1 = Q.qsa_prefill_forward(inp["q"][qs], inp["k"][ks], inp["v"][ks],
                                               inp["q_idx"][qs], inp["w"][qs], inp["k_idx"][ks],
                                               budget=wl.budget, q_pos0=lk - lq, pe=pe)
        torch.cuda.synchronize()
        assert torch.equal(k1, kp[b, : lk // 4]), f"sequence {b}: pooled keys"
        assert torch.equal(s1, sel[qs]) and torch.equal(o1, out[qs]), f"sequence {b}"
