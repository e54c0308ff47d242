"""Decode from a paged K/V cache on an MI355X, through the C ABI: bit for bit against
the contiguous cache, against the oracle through its paged fetcher, and with block
table entries outside the pool (clamped by the kernel, no fault)."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_06_amd as Q
from oracle import qsa_oracle as O
from parity import bits, check_selection_row, compare_output, score_abs_tol, LSE_ABS
from synth import generate, workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _decode_tol(inp, b, t):
    """fp32 score error floor of decode row b (query at position t)."""
    own = t // 4
    return float(score_abs_tol(O.bf16_to_f64(bits(inp["q_idx"][b, 0]))[None],
                               inp["w"][b, 0].double().cpu().numpy()[None],
                               O.bf16_to_f64(bits(inp["k_pooled"][b, :own])), [own])[0])


def _say(*a):
    print(*a, flush=True)


def _paged(kc, vc, P, seed, spare=7):
    """Scatter contiguous caches [B, L, Hkv, d] into pools of shuffled pages (spare pages
    and unused slots hold noise); returns the pools and the block table."""
    bsz, L, hkv, d = kc.shape
    n_per = L // P
    n_pages = bsz * n_per + spare
    g = torch.Generator(device="cpu").manual_seed(seed)
    table = torch.randperm(n_pages, generator=g)[: bsz * n_per].view(bsz, n_per)
    table = table.to(torch.int32).to(DEV)
    gd = torch.Generator(device=DEV).manual_seed(seed)
    k_pool = torch.randn((n_pages * P, hkv, d), generator=gd, device=DEV).to(torch.bfloat16)
    v_pool = torch.randn((n_pages * P, hkv, d), generator=gd, device=DEV).to(torch.bfloat16)
    slots = (table.long()[:, :, None] * P + torch.arange(P, device=DEV)).reshape(-1)
    k_pool[slots] = kc.reshape(-1, hkv, d)
    v_pool[slots] = vc.reshape(-1, hkv, d)
    return k_pool, v_pool, table


def _inputs(seq, lk=65536):
    wl = workload("decode1m", batch=len(seq), lk=lk)
    return wl, generate(wl, device=DEV, seq_lens=seq)


def _decode(inp, wl, paged=None, P=None):
    if paged is None:
        return Q.qsa_decode_forward(inp["q"], inp["q_idx"], inp["w"], inp["k_pooled"],
                                    inp["k_cache"], inp["v_cache"], inp["seq_lens"],
                                    budget=wl.budget)
    k_pool, v_pool, table = paged
    return Q.qsa_decode_forward_paged(inp["q"], inp["q_idx"], inp["w"], inp["k_pooled"], k_pool,
                                      v_pool, table, inp["seq_lens"], budget=wl.budget,
                                      page_size=P, lmax=wl.lk)


@pytest.mark.parametrize("P", [4, 64, 256])
def test_paged_decode_equals_contiguous(P):
    seq = [65536, 40001, 1500, 9]
    _say(f"paged decode P={P} seq={seq}")
    wl, inp = _inputs(seq)
    ref = [t.clone() for t in _decode(inp, wl)]
    got = _decode(inp, wl, _paged(inp["k_cache"], inp["v_cache"], P, seed=P), P)
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "lse", "sel"), got, ref):
        assert torch.equal(a, b), f"{name} differs from the contiguous cache (P={P})"


def test_paged_decode_against_oracle():
    seq = [65536, 33333, 2048, 100]
    P = 16
    _say(f"paged decode vs oracle P={P} seq={seq}")
    wl, inp = _inputs(seq)
    k_pool, v_pool, table = _paged(inp["k_cache"], inp["v_cache"], P, seed=3)
    out, lse, sel = _decode(inp, wl, (k_pool, v_pool, table), P)
    torch.cuda.synchronize()
    fetch = O.paged_fetcher(bits(k_pool), bits(v_pool), table.cpu().numpy(), P)
    res = O.forward_decode(bits(inp["q"]), bits(inp["q_idx"])[:, 0], inp["w"].cpu().numpy()[:, 0],
                           bits(inp["k_pooled"]), np.array(seq), fetch, r=4, budget=wl.budget)
    sel_np = sel.cpu().numpy()
    for b in range(len(seq)):
        t = seq[b] - 1
        check_selection_row(sel_np[b], res["scores"][b], t // 4, wl.n_sel, f"paged b={b}",
                            abs_tol=_decode_tol(inp, b, t))
        kr, vr = fetch(b, O.kept_tokens(sel_np[b], t, 4, t + 1))
        ref, ref_lse = O.attend(O.bf16_to_f64(bits(inp["q"][b])), kr, vr, 1 / math.sqrt(wl.d))
        compare_output(out[b], ref, f"paged b={b}")
        assert np.max(np.abs(lse[b].double().cpu().numpy() - ref_lse)) <= LSE_ABS


def test_paged_table_entries_outside_the_pool_are_clamped():
    seq = [8192, 4096]
    P = 64
    wl, inp = _inputs(seq, lk=8192)
    k_pool, v_pool, table = _paged(inp["k_cache"], inp["v_cache"], P, seed=5)
    table[0, ::3] = -3
    table[1, 1::2] = k_pool.shape[0] // P + 100
    out, lse, sel = _decode(inp, wl, (k_pool, v_pool, table), P)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
