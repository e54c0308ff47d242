"""Parity of the indexer warm-up kernels (through the C ABI) with the CPU oracle:
the dense KL target, the KL loss with its score gradient, and the indexer's
backward (with the pooling's)."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_06_amd as Q
from oracle import qsa_oracle as O
from parity import bits, compare_grad

pytestmark = pytest.mark.gpu

DEV = "cuda"
TARGET_REL = 1e-4   # fp32 MFMA sums of exact bf16 products, fp32 exp: ~1e-6 relative
LSE_TOL = 1e-4
LOSS_REL = 1e-4


def _say(*a):
    print(*a, flush=True)


def _randn_bf16(shape, seed, scale=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(torch.bfloat16)


def _target_case(lq, lk, q_pos0, hq, hkv, d, seed, unscaled=False):
    sc = 1.0 if unscaled else 1 / math.sqrt(d)
    q = _randn_bf16((lq, hq, d), seed, sc)
    k = _randn_bf16((lk, hkv, d), seed + 1, sc)
    _say(f"kl target lq={lq} lk={lk} q_pos0={q_pos0} heads={hq}/{hkv} d={d}")
    lse, target = Q.qsa_indexer_kl_target(q, k, q_pos0=q_pos0)
    torch.cuda.synchronize()
    qf, kf = O.bf16_to_f64(bits(q)), O.bf16_to_f64(bits(k))
    lse_g, tg = lse.double().cpu().numpy(), target.double().cpu().numpy()
    scale = 1 / math.sqrt(d)
    worst_t, worst_l = 0.0, 0.0
    for i in range(lq):
        t = q_pos0 + i
        ref = O.kl_block_target(qf[i], kf[: t + 1], t, 4, scale)
        _, lse_ref = O.attend(qf[i], kf[: t + 1], kf[: t + 1], scale)
        worst_l = max(worst_l, float(np.abs(lse_g[i] - lse_ref).max()))
        if ref.size:
            got = tg[i, : ref.size]
            got = got / got.sum()
            worst_t = max(worst_t, float(np.abs(got - ref).max() / ref.max()))
    _say(f"  lse max abs {worst_l:.2e}; target max rel {worst_t:.2e}")
    assert worst_l <= LSE_TOL
    assert worst_t <= TARGET_REL
    return q, k, lse, target


def test_kl_target_small_ragged():
    _target_case(lq=300, lk=501, q_pos0=201, hq=4, hkv=2, d=128, seed=60)


def test_kl_target_model_shape_and_peaky():
    _target_case(lq=128, lk=2176, q_pos0=2048, hq=24, hkv=2, d=256, seed=61)
    _target_case(lq=96, lk=700, q_pos0=604, hq=6, hkv=2, d=128, seed=62, unscaled=True)


def test_kl_target_more_groups():
    # 3 and 4 KV groups take the one-row-per-wave shape; 1 group the two-row one.
    _target_case(lq=37, lk=300, q_pos0=263, hq=12, hkv=3, d=256, seed=67)
    _target_case(lq=70, lk=150, q_pos0=80, hq=16, hkv=4, d=128, seed=68)
    _target_case(lq=33, lk=33, q_pos0=0, hq=16, hkv=1, d=128, seed=69)


def test_kl_loss_and_score_gradient():
    # The loss kernel on the GPU's own scores and target, against the oracle on the same
    # numbers; then end to end against the oracle's own scores and target.
    lq, lk, q_pos0, hq, hkv, d, hi, di = 200, 1100, 900, 4, 1, 128, 4, 128
    q, k, _, target = _target_case(lq, lk, q_pos0, hq, hkv, d, seed=63)
    qi = _randn_bf16((lq, hi, di), 64, 1 / math.sqrt(di))
    ki = _randn_bf16((lk, di), 65, 1 / math.sqrt(di))
    g = torch.Generator(device=DEV)
    g.manual_seed(66)
    w = torch.rand((lq, hi), generator=g, device=DEV)
    kp = Q.qsa_pool_keys(ki)
    nblk = lk // 4
    scores = Q.qsa_index_scores(qi, w, kp, q_pos0=q_pos0)
    loss, ds = Q.qsa_indexer_kl_loss(scores, target, nblk=nblk, q_pos0=q_pos0)
    torch.cuda.synchronize()
    s_g, t_g = scores.double().cpu().numpy(), target.double().cpu().numpy()
    loss_g, ds_g = loss.double().cpu().numpy(), ds.double().cpu().numpy()
    sc_ref = O.index_scores(O.bf16_to_f64(bits(qi)), w.double().cpu().numpy(),
                            O.bf16_to_f64(bits(kp)), q_pos0 + np.arange(lq), 4)
    qf, kf = O.bf16_to_f64(bits(q)), O.bf16_to_f64(bits(k))
    worst_same, worst_e2e, worst_ds = 0.0, 0.0, 0.0
    for i in range(lq):
        t = q_pos0 + i
        n = min(t // 4, nblk)
        p_same = t_g[i, :n] / t_g[i, :n].sum()
        l_same, d_same = O.indexer_kl(s_g[i, :n], p_same)
        worst_same = max(worst_same, abs(loss_g[i] - l_same) / max(abs(l_same), 1e-6))
        worst_ds = max(worst_ds, float(np.abs(ds_g[i, :n] - d_same).max()))
        l_ref, _ = O.indexer_kl(sc_ref[i, :n], O.kl_block_target(qf[i], kf[: t + 1], t, 4,
                                                                 1 / math.sqrt(d)))
        worst_e2e = max(worst_e2e, abs(loss_g[i] - l_ref) / max(abs(l_ref), 1e-6))
    _say(f"  loss rel (same inputs) {worst_same:.2e}, ds abs {worst_ds:.2e}, "
         f"loss rel (end to end) {worst_e2e:.2e}")
    assert worst_same <= 1e-5
    assert worst_ds <= 1e-7
    assert worst_e2e <= LOSS_REL


def test_kl_loss_rows_without_scored_blocks():
    # Rows at t < r score nothing: loss 0.
    lq, lk = 40, 40
    q = _randn_bf16((lq, 2, 128), 67, 1 / math.sqrt(128))
    k = _randn_bf16((lk, 1, 128), 68, 1 / math.sqrt(128))
    _, target = Q.qsa_indexer_kl_target(q, k, q_pos0=0)
    scores = torch.zeros_like(target)
    loss, _ = Q.qsa_indexer_kl_loss(scores, target, nblk=lk // 4, q_pos0=0)
    torch.cuda.synchronize()
    assert torch.all(loss[:4] == 0)
    assert torch.all(loss[4:] >= -1e-6)


@pytest.mark.parametrize("hi,di,lq,q_pos0,lk", [(4, 128, 300, 201, 501), (3, 64, 130, 0, 130)])
def test_index_scores_backward(hi, di, lq, q_pos0, lk):
    qi = _randn_bf16((lq, hi, di), 70, 1 / math.sqrt(di))
    ki = _randn_bf16((lk, di), 71, 1 / math.sqrt(di))
    g = torch.Generator(device=DEV)
    g.manual_seed(72)
    w = torch.rand((lq, hi), generator=g, device=DEV)
    kp = Q.qsa_pool_keys(ki)
    nblk = lk // 4
    ld = Q.score_ld(nblk)
    ds_np = np.random.default_rng(73).standard_normal((lq, ld)).astype(np.float32)
    own = (q_pos0 + np.arange(lq)) // 4
    ds_np[np.arange(ld)[None, :] >= np.minimum(own, nblk)[:, None]] = np.nan  # never read
    ds = torch.from_numpy(ds_np).to(DEV)
    _say(f"index scores backward H_I={hi} d_I={di} lq={lq} q_pos0={q_pos0} lk={lk}")
    dq, dw, dkp, dki = Q.qsa_index_scores_bwd(qi, w, kp, ds, q_pos0=q_pos0, n_tokens=lk)
    torch.cuda.synchronize()
    rq, rw, rk = O.index_scores_backward(O.bf16_to_f64(bits(qi)), w.double().cpu().numpy(),
                                         O.bf16_to_f64(bits(kp)), ds_np[:, :nblk].astype(np.float64),
                                         q_pos0 + np.arange(lq), 4)
    for name, got, ref in (("dq_idx", dq, rq), ("dk_pooled", dkp, rk)):
        mx, rel = compare_grad(got, ref, name)
        _say(f"  {name}: max-abs/max|ref| {mx:.2e}  rel-L2 {rel:.2e}")
    dw_err = float(np.abs(dw.double().cpu().numpy() - rw).max() / np.abs(rw).max())
    _say(f"  dw max rel {dw_err:.2e}")
    assert dw_err <= 1e-5  # fp32 z and ds: no bf16 operand on this path
    ref_ki = O.pool_keys_backward(dkp.double().cpu().numpy(), 4, lk)
    np.testing.assert_allclose(dki.double().cpu().numpy(), ref_ki, rtol=1e-6, atol=0)
