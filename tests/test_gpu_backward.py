"""Parity of the sparse-attention backward (through the C ABI) with the CPU oracle.

Each case runs the GPU forward for out and lse, then the GPU backward, and compares
dq, dk and dv element by element with the oracle's fp64 gradients on the same bf16
inputs and the same selections.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_06_amd as Q
from oracle import qsa_oracle as O
from parity import bits, compare_grad

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


def _randn_bf16(shape, seed, scale=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(torch.bfloat16)


def _random_selection(rows_t, n_sel, r, seed):
    """Valid selections (ascending, own block last, -1 padded), random earlier blocks."""
    rng = np.random.default_rng(seed)
    sel = np.full((len(rows_t), n_sel), -1, dtype=np.int32)
    for i, t in enumerate(rows_t):
        own = int(t) // r
        m = min(n_sel - 1, own)
        pick = np.sort(rng.choice(own, size=m, replace=False)) if m else np.zeros(0, int)
        sel[i, :m] = pick
        sel[i, m] = own
    return sel


def _case(lq, lk, q_pos0, hq, hkv, d, budget, seed, unscaled=False):
    sc = 1.0 if unscaled else 1 / math.sqrt(d)
    q = _randn_bf16((lq, hq, d), seed, sc)
    k = _randn_bf16((lk, hkv, d), seed + 1, sc)
    v = _randn_bf16((lk, hkv, d), seed + 2, 1 / math.sqrt(d))
    dout = _randn_bf16((lq, hq, d), seed + 3)
    sel_np = _random_selection(q_pos0 + np.arange(lq), budget // 4, 4, seed)
    sel = torch.from_numpy(sel_np).to(DEV)
    _say(f"backward lq={lq} lk={lk} q_pos0={q_pos0} heads={hq}/{hkv} d={d} budget={budget}")
    out, lse = Q.qsa_sparse_attn_fwd(q, k, v, sel, q_pos0=q_pos0)
    dq, dk, dv = Q.qsa_sparse_attn_bwd(q, k, v, sel, out, lse, dout, q_pos0=q_pos0)
    torch.cuda.synchronize()
    ref = O.backward_prefill(bits(q), bits(k), bits(v), sel_np,
                             O.bf16_to_f64(bits(dout)), r=4, q_pos0=q_pos0,
                             scale=1 / math.sqrt(d))
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        mx, rel = compare_grad(got, ref[name], f"{name} lq={lq} d={d}")
        _say(f"  {name}: max-abs/max|ref| {mx:.2e}  rel-L2 {rel:.2e}")
    return (q, k, v, sel, out, lse, dout), (dq, dk, dv)


def test_backward_small_ragged():
    # 501 keys: the last key block is partial and is the own block of the last rows.
    _case(lq=300, lk=501, q_pos0=201, hq=4, hkv=2, d=128, budget=64, seed=40)


def test_backward_model_shape():
    _case(lq=256, lk=3256, q_pos0=3000, hq=24, hkv=2, d=256, budget=2048, seed=41)


def test_backward_early_rows_dense_and_deterministic():
    # Rows before the budget read every earlier token (dense causal attention).
    args, grads = _case(lq=600, lk=600, q_pos0=0, hq=8, hkv=1, d=128, budget=512, seed=42)
    again = Q.qsa_sparse_attn_bwd(*args[:4], args[4], args[5], args[6], q_pos0=0)
    torch.cuda.synchronize()
    for a, b in zip(grads, again):
        assert torch.equal(a, b), "backward is not bit-reproducible"


def test_backward_softmax_stress():
    # Unscaled N(0,1) q and k: peaky softmax rows.
    _case(lq=200, lk=1200, q_pos0=1000, hq=6, hkv=2, d=128, budget=256, seed=43,
          unscaled=True)


@pytest.mark.parametrize("hq,hkv", [(10, 2), (16, 1)])
def test_backward_head_group_sizes(hq, hkv):
    # 5 heads per group: a row's group spans 2.5 KiB, the last 1 KiB load half used;
    # 16 heads: every tile row is a real head.
    _case(lq=160, lk=900, q_pos0=740, hq=hq, hkv=hkv, d=256, budget=512, seed=44 + hq)
