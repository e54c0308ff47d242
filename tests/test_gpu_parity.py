"""Parity of the HIP path (through the C ABI) with the CPU oracle, on an MI355X.

Small cases compare every element; the full-size workloads run in the launch
configuration of bench.py and compare sampled rows the oracle computes one by one.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_06_amd as Q
from oracle import qsa_oracle as O
from parity import bits, check_selection_row, compare_output, score_abs_tol, LSE_ABS, SCORE_REL
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


def _randn_bf16(shape, seed, scale=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(torch.bfloat16)


def _random_selection(rows_t, n_sel, r, seed, nblk_cap=None):
    """Valid selections (ascending, own last, -1 padded) with random earlier blocks."""
    rng = np.random.default_rng(seed)
    sel = np.full((len(rows_t), n_sel), -1, dtype=np.int32)
    for i, t in enumerate(rows_t):
        own = int(t) // r
        cand = own if nblk_cap is None else min(own, nblk_cap)
        m = min(n_sel - 1, cand)
        pick = np.sort(rng.choice(cand, size=m, replace=False)) if m else np.zeros(0, int)
        sel[i, :m] = pick
        sel[i, m] = own
    return sel


# ------------------------------------------------------------------------------------
# Stage 1: pooling (bit-exact)
# ------------------------------------------------------------------------------------


@pytest.mark.parametrize("n_tok,d_i,row_stride", [(2048, 64, 64), (4 * 1000 + 3, 128, 128),
                                                  (8, 128, 256), (4 * 777, 128, 136)])
def test_pool_keys_bit_exact(n_tok, d_i, row_stride):
    _say(f"pool n_tok={n_tok} d_i={d_i} stride={row_stride}")
    base = _randn_bf16((n_tok, row_stride), seed=n_tok, scale=1 / math.sqrt(d_i))
    k = base[:, :d_i]
    out = Q.qsa_pool_keys(k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), O.pool_keys(bits(k), 4))


@pytest.mark.parametrize("n_tok,d_i", [(4 * 300 + 3, 256), (4 * 200, 512), (4 * 513 + 2, 96),
                                      (4 * 100 + 1, 1024), (4 * 50, 8), (4 * 70, 32)])
def test_pool_keys_other_widths(n_tok, d_i):
    # widths whose rows fill whole waves (8..512) and widths that do not (96, 1024)
    _say(f"pool n_tok={n_tok} d_i={d_i}")
    k = _randn_bf16((n_tok, d_i), seed=n_tok + d_i, scale=1 / math.sqrt(d_i))
    out = Q.qsa_pool_keys(k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), O.pool_keys(bits(k), 4))


# ------------------------------------------------------------------------------------
# Stage 2: scores
# ------------------------------------------------------------------------------------


def _score_bound(q, w, kp):
    """Magnitude of the summed terms (for the fp32-accumulation tolerance)."""
    tot = 0
    for h in range(q.shape[1]):
        tot = tot + np.abs(w[:, h : h + 1]) * (np.abs(q[:, h, :]) @ np.abs(kp).T)
    return tot


@pytest.mark.parametrize("lq,q_pos0,nblk,h_i,d_i", [(2048, 0, 512, 4, 64), (333, 4 * 97 + 1, 300, 3, 128),
                                                     (130, 8192, 2100, 4, 128), (64, 5, 40, 1, 64)])
def test_index_scores(lq, q_pos0, nblk, h_i, d_i):
    _say(f"scores lq={lq} q_pos0={q_pos0} nblk={nblk} h_i={h_i} d_i={d_i}")
    q = _randn_bf16((lq, h_i, d_i), 1, 1 / math.sqrt(d_i))
    kp = _randn_bf16((nblk, d_i), 2, 0.5 / math.sqrt(d_i))
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    w = torch.rand((lq, h_i), generator=g, device=DEV)
    w[::7] *= -1.0  # negative weights too
    s = Q.qsa_index_scores(q, w, kp, q_pos0=q_pos0)
    torch.cuda.synchronize()
    qf, kf, wf = O.bf16_to_f64(bits(q)), O.bf16_to_f64(bits(kp)), w.double().cpu().numpy()
    pos = q_pos0 + np.arange(lq)
    ref = O.index_scores(qf, wf, kf, pos, 4)
    bound = _score_bound(qf, wf, kf)
    got = s.double().cpu().numpy()[:, :nblk]
    own = np.minimum(pos // 4, nblk)
    mask = np.arange(nblk)[None, :] < own[:, None]
    err = np.abs(got - np.nan_to_num(ref))[mask]
    assert np.all(err <= SCORE_REL * bound[mask] + 1e-30), f"max err {err.max()}"


def test_index_scores_batched_seq_lens():
    bsz, lq, h_i, d_i, nblk = 3, 5, 4, 128, 256
    seq = [1024, 997, 23]
    _say(f"scores batched seq_lens={seq}")
    q = _randn_bf16((bsz, lq, h_i, d_i), 4, 1 / math.sqrt(d_i))
    kp = _randn_bf16((bsz, nblk, d_i), 5, 1 / math.sqrt(d_i))
    w = torch.rand((bsz, lq, h_i), device=DEV)
    sl = torch.tensor(seq, dtype=torch.int32, device=DEV)
    s = Q.qsa_index_scores(q, w, kp, seq_lens=sl)
    torch.cuda.synchronize()
    for b in range(bsz):
        pos = seq[b] - lq + np.arange(lq)
        qf, kf, wf = O.bf16_to_f64(bits(q[b])), O.bf16_to_f64(bits(kp[b])), w[b].double().cpu().numpy()
        ref = O.index_scores(qf, wf, kf, pos, 4)
        bound = _score_bound(qf, wf, kf)
        got = s[b].double().cpu().numpy()[:, :nblk]
        for i in range(lq):
            own = max(0, min(pos[i] // 4, nblk)) if pos[i] >= 0 else 0
            assert np.all(np.abs(got[i, :own] - ref[i, :own]) <= SCORE_REL * bound[i, :own] + 1e-30)


@pytest.mark.parametrize("d_i,h_i,lq,seq", [(128, 4, 4, [800_003, 333_337, 4093, 5]),
                                             (64, 3, 1, [262_147, 1_000_000, 65, 4])])
def test_index_scores_streaming_scan(d_i, h_i, lq, seq):
    """Few rows per sequence take the streaming scan: long ranges split into several
    chunks per wave, ragged ends, rows with no block to score."""
    bsz = len(seq)
    nblk = max(seq) // 4
    _say(f"scores scan lq={lq} d_i={d_i} seq_lens={seq}")
    q = _randn_bf16((bsz, lq, h_i, d_i), 6, 1 / math.sqrt(d_i))
    kp = _randn_bf16((bsz, nblk, d_i), 7, 1 / math.sqrt(d_i))
    g = torch.Generator(device=DEV)
    g.manual_seed(8)
    w = torch.rand((bsz, lq, h_i), generator=g, device=DEV) - 0.3
    sl = torch.tensor(seq, dtype=torch.int32, device=DEV)
    s = Q.qsa_index_scores(q, w, kp, seq_lens=sl)
    torch.cuda.synchronize()
    for b in range(bsz):
        pos = seq[b] - lq + np.arange(lq)
        qf, kf, wf = O.bf16_to_f64(bits(q[b])), O.bf16_to_f64(bits(kp[b])), w[b].double().cpu().numpy()
        ref = O.index_scores(qf, wf, kf, pos, 4)
        bound = _score_bound(qf, wf, kf)
        got = s[b].double().cpu().numpy()[:, :nblk]
        for i in range(lq):
            own = max(0, min(pos[i] // 4, nblk)) if pos[i] >= 0 else 0
            assert np.all(np.abs(got[i, :own] - ref[i, :own]) <= SCORE_REL * bound[i, :own] + 1e-30)


# ------------------------------------------------------------------------------------
# Stage 3: top-k on given scores (same fp32 inputs on both sides: exact equality)
# ------------------------------------------------------------------------------------


def _run_topk(scores_np, q_pos0, nblk, budget, seq_lens=None):
    lq = scores_np.shape[-2] if scores_np.ndim == 3 else scores_np.shape[0]
    ld = Q.score_ld(nblk)
    shp = (scores_np.shape[0], lq, ld) if scores_np.ndim == 3 else (lq, ld)
    full = np.full(shp, np.nan, dtype=np.float32)  # never-read entries are NaN
    full[..., : scores_np.shape[-1]] = scores_np
    st = torch.from_numpy(full).to(DEV)
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    sel = Q.qsa_topk_blocks(st, lq=lq, nblk=nblk, budget=budget, q_pos0=q_pos0, seq_lens=sl)
    torch.cuda.synchronize()
    return sel.cpu().numpy()


def _check_topk_exact(scores_np, sel, q_pos0, nblk, n_sel, r=4):
    for i in range(sel.shape[0]):
        t = q_pos0 + i
        own = t // r
        c = min(own, nblk)  # candidates stop at the pooled range; own block still kept
        m = min(n_sel - 1, c)
        ranked = O.select_blocks(scores_np[i, :c].astype(np.float64), c, n_sel)
        ref = np.full(n_sel, -1)
        ref[:m] = ranked[:m]
        ref[m] = own
        np.testing.assert_array_equal(sel[i], ref, err_msg=f"row {i} (t={t})")


def _nan_tail(x, q_pos0, r=4):
    x = x.copy()
    for i in range(x.shape[0]):
        x[i, (q_pos0 + i) // r :] = np.nan
    return x


@pytest.mark.parametrize("kind", ["normal", "quantized", "zeros_negzero", "negative", "relu_like"])
def test_topk_exact(kind):
    rng = np.random.default_rng(11)
    lq, q_pos0, budget = 257, 4 * 300 + 2, 256  # n_sel = 64; rows 300..364 blocks
    nblk = (q_pos0 + lq) // 4 + 1
    x = rng.standard_normal((lq, nblk)).astype(np.float32)
    if kind == "quantized":
        x = np.round(x * 2) / 2
    elif kind == "zeros_negzero":
        x = np.where(rng.random(x.shape) < 0.5, np.float32(0.0), np.float32(-0.0))
        x[:, ::37] = 1.0
    elif kind == "negative":
        x = -np.abs(x)
    elif kind == "relu_like":
        x = np.maximum(x, 0) * rng.random(x.shape).astype(np.float32)
    _say(f"topk kind={kind}")
    sel = _run_topk(_nan_tail(x, q_pos0), q_pos0, nblk, budget)
    _check_topk_exact(x, sel, q_pos0, nblk, budget // 4)


def test_topk_short_rows_and_nblk_cap():
    rng = np.random.default_rng(12)
    lq, q_pos0, budget, nblk = 300, 0, 128, 50  # rows beyond block 50: candidates capped
    x = rng.standard_normal((lq, nblk)).astype(np.float32)
    _say("topk short rows / nblk cap")
    sel = _run_topk(x, q_pos0, nblk, budget)
    _check_topk_exact(x, sel, q_pos0, nblk, budget // 4)


def test_topk_huge_tie_set_takes_lowest_ids():
    # 20000 candidates, 100 positive, the rest exactly zero: the 411 zeros kept are
    # the lowest ids (exercises the in-order path beyond the LDS tie capacity).
    lq, budget = 2, 2048
    q_pos0 = 4 * 20000
    nblk = 20001
    x = np.zeros((lq, nblk), dtype=np.float32)
    pos = np.random.default_rng(13).choice(20000, 100, replace=False)
    x[:, pos] = 1.0 + np.arange(100, dtype=np.float32)
    x[1, 5::2] = -0.0
    _say("topk huge tie set")
    sel = _run_topk(_nan_tail(x, q_pos0), q_pos0, nblk, budget)
    _check_topk_exact(x, sel, q_pos0, nblk, budget // 4)


@pytest.mark.parametrize("pattern", ["runs32_every16", "runs32_every8"])
@pytest.mark.parametrize("sampled_high", [True, False])
def test_topk_adversarial_sample(pattern, sampled_high):
    # A row of 32768 candidates is sampled at 64 evenly spaced runs of 32 scores (every
    # 16th run). Large values only in the sampled runs make the threshold too high
    # (fewer than m candidates pass); only outside them, too low (the candidate list
    # overflows). Both must fall back to the exact selection over the whole row. The
    # runs32_every8 pattern (a superset of the sampled runs) is a second spacing.
    rng = np.random.default_rng(15 + sampled_high)
    lq, budget = 3, 2048
    q_pos0 = 4 * 32768
    nblk = 32768 + 4
    x = rng.random((lq, nblk)).astype(np.float32)
    if pattern == "runs32_every16":
        sampled = (np.arange(nblk) // 32) % 16 == 0
    else:
        sampled = (np.arange(nblk) // 32) % 8 == 0
    hi = sampled if sampled_high else ~sampled
    x[:, hi] += 10.0
    _say(f"topk adversarial pattern={pattern} sampled_high={sampled_high}")
    sel = _run_topk(_nan_tail(x, q_pos0), q_pos0, nblk, budget)
    _check_topk_exact(x, sel, q_pos0, nblk, budget // 4)


@pytest.mark.parametrize("budget", [2048, 4096, 64])
@pytest.mark.parametrize("kind", ["normal", "quantized"])
def test_topk_row_lengths_around_the_list_size(budget, kind):
    # Rows just below, at and above the list size (1664 entries for budgets up to
    # 2048, else 2048: every score is a list entry up to that; longer rows are sampled),
    # a ragged length and the 32768 maximum, with distinct scores and with heavy ties
    # (quantized to halves).
    rng = np.random.default_rng(budget + len(kind))
    for c0 in (1662, 1664, 2046, 2047, 2048, 2049, 5001, 32760):
        q_pos0, lq = 4 * c0 + 1, 8
        nblk = min((q_pos0 + lq) // 4 + 1, 32768)
        x = rng.standard_normal((lq, nblk)).astype(np.float32)
        if kind == "quantized":
            x = np.round(x * 2) / 2
        _say(f"topk rows from {c0} blocks, budget {budget}, {kind}")
        sel = _run_topk(_nan_tail(x, q_pos0), q_pos0, nblk, budget)
        _check_topk_exact(x, sel, q_pos0, nblk, budget // 4)


@pytest.mark.parametrize("q_blk,lq,nblk,budget,kind",
                         [(69000, 700, 70000, 2048, "normal"), (69000, 700, 70000, 4096, "quantized"),
                          (32500, 2100, 33100, 2048, "quantized")])
def test_topk_long_rows_by_waves(q_blk, lq, nblk, budget, kind):
    # Enough rows of more than 32768 candidates to take the two wave passes (best of
    # each 32768-score segment, then best of the kept): three segments with a ragged
    # last one, heavy ties, and rows on both sides of 32768 candidates in one launch.
    rng = np.random.default_rng(q_blk + budget)
    q_pos0 = 4 * q_blk + 3
    x = rng.standard_normal((lq, nblk)).astype(np.float32)
    if kind == "quantized":
        x = np.round(x * 2) / 2
    _say(f"topk long rows by waves: rows {lq}, from {q_blk} blocks, budget {budget}, {kind}")
    sel = _run_topk(_nan_tail(x, q_pos0), q_pos0, nblk, budget)
    _check_topk_exact(x, sel, q_pos0, nblk, budget // 4)


def test_topk_long_rows_concentrated_best():
    # Rows longer than one workgroup's 32768 candidates are split into segments that
    # each keep only a few candidates. Here every one of the best blocks sits in one
    # segment (and, in the second row, the scores rise with the block id), so the
    # merge must notice the truncation and redo the selection over the whole row.
    rng = np.random.default_rng(16)
    bsz, nblk, budget = 2, 262144, 2048
    seq = [1048576, 1048576 - 4 * 1000]
    x = rng.random((bsz, 1, nblk)).astype(np.float32)
    x[0, 0, 100000:100600] += 5.0
    x[1, 0, :] = np.arange(nblk, dtype=np.float32) / nblk
    _say("topk long rows, concentrated best")
    sel = _run_topk(x, 0, nblk, budget, seq_lens=seq)
    for b in range(bsz):
        t = seq[b] - 1
        own = t // 4
        ref = O.select_blocks(x[b, 0, :own].astype(np.float64), own, budget // 4)
        np.testing.assert_array_equal(sel[b, 0], ref)


def test_topk_decode_rows_batched():
    rng = np.random.default_rng(14)
    bsz, nblk, budget = 3, 262144, 2048
    seq = [1048576, 1048573, 4 * 100000 + 1]
    x = np.maximum(rng.standard_normal((bsz, 1, nblk)).astype(np.float32), 0)
    _say("topk decode rows 262K")
    sel = _run_topk(x, 0, nblk, budget, seq_lens=seq)
    for b in range(bsz):
        t = seq[b] - 1
        own = t // 4
        ref = O.select_blocks(x[b, 0, :own].astype(np.float64), own, budget // 4)
        np.testing.assert_array_equal(sel[b, 0], ref)


@pytest.mark.parametrize("budget", [2048, 4096])
def test_topk_merge_short_and_tied_rows(budget):
    # Rows of a long launch (262144 pooled blocks: the two-pass top-k runs) that the
    # segment winners cannot settle: fewer candidates than places (a short sequence,
    # and with budget 4096 also a row just past one workgroup's 32768 candidates),
    # and a row of equal scores (one value bin holds every candidate; the lowest ids
    # win). The last row is ordinary.
    rng = np.random.default_rng(17)
    nblk = 262144
    seq = [5000, 4 * 33000 + 3, 1048576, 1048576 - 77]
    x = rng.random((len(seq), 1, nblk)).astype(np.float32)
    x[2, 0, :] = 0.5
    _say(f"topk merge short and tied rows, budget {budget}")
    sel = _run_topk(x, 0, nblk, budget, seq_lens=seq)
    for b in range(len(seq)):
        own = (seq[b] - 1) // 4
        ref = O.select_blocks(x[b, 0, :own].astype(np.float64), own, budget // 4)
        np.testing.assert_array_equal(sel[b, 0], ref, err_msg=f"row {b} (seq {seq[b]})")


# ------------------------------------------------------------------------------------
# Stage 4: attention on given selections
# ------------------------------------------------------------------------------------


def _attn_case(lq, lk, q_pos0, hq, hkv, d, budget, seed, unscaled=False, rows=None,
               sel_offset=0):
    sc = 1.0 if unscaled else 1 / math.sqrt(d)
    q = _randn_bf16((lq, hq, d), seed, sc)
    k = _randn_bf16((lk, hkv, d), seed + 1, sc)
    v = _randn_bf16((lk, hkv, d), seed + 2, 1 / math.sqrt(d))
    pos = q_pos0 + np.arange(lq)
    n_sel = budget // 4
    sel_np = _random_selection(pos, n_sel, 4, seed)
    if sel_offset:
        # A contiguous view that starts sel_offset int32s into its allocation.
        buf = torch.full((lq * n_sel + sel_offset,), -1, dtype=torch.int32, device=DEV)
        sel = buf[sel_offset:].view(lq, n_sel)
        sel.copy_(torch.from_numpy(sel_np))
    else:
        sel = torch.from_numpy(sel_np).to(DEV)
    out, lse = Q.qsa_sparse_attn_fwd(q, k, v, sel, q_pos0=q_pos0)
    torch.cuda.synchronize()
    rows = np.arange(lq) if rows is None else np.asarray(rows)
    qb, kb, vb = bits(q), bits(k), bits(v)
    ref = np.zeros((len(rows), hq, d))
    ref_lse = np.zeros((len(rows), hq))
    for j, i in enumerate(rows):
        toks = O.kept_tokens(sel_np[i], int(pos[i]), 4, lk)
        ref[j], ref_lse[j] = O.attend(O.bf16_to_f64(qb[i]), O.bf16_to_f64(kb[toks]),
                                      O.bf16_to_f64(vb[toks]), 1 / math.sqrt(d))
    compare_output(out[torch.from_numpy(rows).to(DEV)], ref, f"attn lq={lq} d={d}")
    got_lse = lse.double().cpu().numpy()[rows]
    assert np.max(np.abs(got_lse - ref_lse)) <= LSE_ABS


@pytest.mark.parametrize("lq,lk,q_pos0,hq,hkv,d,budget", [
    (2048, 2048, 0, 4, 1, 128, 256),            # tiny shape
    (700, 4102, 3402, 24, 2, 256, 2048),        # model shape, ragged Lk, chunk at the end
    (513, 513, 0, 16, 1, 256, 64),              # 16 heads per group, partial last block
    (300, 1200, 900, 2, 2, 128, 16),            # 1 head per group, few blocks
])
def test_sparse_attn_fwd(lq, lk, q_pos0, hq, hkv, d, budget):
    _say(f"attn lq={lq} lk={lk} q_pos0={q_pos0} hq={hq} hkv={hkv} d={d} K={budget}")
    _attn_case(lq, lk, q_pos0, hq, hkv, d, budget, seed=lq)


@pytest.mark.parametrize("budget,sel_offset", [
    (52, 0),    # 13 blocks a row: rows are not a whole number of 16-byte id groups
    (28, 1),    # 7 blocks a row, rows start 4 bytes past a 16-byte boundary
    (256, 1),   # 64 blocks a row, every row start off a 16-byte boundary
])
def test_sparse_attn_fwd_unaligned_selection_rows(budget, sel_offset):
    # The attention reads a step's four block ids 16 bytes at once only when every row
    # starts on a 16-byte boundary; other selection layouts take the id-by-id reads.
    _say(f"attn selection rows K={budget} offset={sel_offset}")
    _attn_case(400, 1500, 1100, 24, 2, 256, budget, seed=budget + sel_offset,
               sel_offset=sel_offset)


@pytest.mark.parametrize("lq,lk,q_pos0,hq,hkv,d", [
    (2500, 70000, 67500, 24, 2, 256),   # K/V 143 MB: one KV group per launch
    (3000, 140000, 137000, 8, 2, 128),  # the same order at d = 128
])
def test_sparse_attn_fwd_group_by_group(lq, lk, q_pos0, hq, hkv, d):
    # Contexts whose K/V exceed 128 MB run one KV group at a time, in launches of one
    # resident generation of rows (2048 here): rows on both sides of a launch edge, the
    # ragged last launch and random rows, checked against the oracle.
    _say(f"attn by group lq={lq} lk={lk} hq={hq} hkv={hkv} d={d}")
    rng = np.random.default_rng(lq)
    rows = np.unique(np.concatenate([[0, 1, 2046, 2047, 2048, 2049, lq - 1],
                                     rng.integers(0, lq, 25)]))
    _attn_case(lq, lk, q_pos0, hq, hkv, d, 2048, seed=lq + 5, rows=rows)


def test_sparse_attn_fwd_softmax_stress():
    # Unscaled N(0,1) q/k with scale 1/sqrt(d): peaky logits, exercises the rescaling.
    _say("attn softmax stress")
    _attn_case(600, 600, 0, 24, 2, 256, 512, seed=77, unscaled=True)


@pytest.mark.parametrize("lmax,hq,hkv,d,budget,seq", [
    (5000, 24, 2, 256, 2048, [5000, 4093, 17]),      # model shape: 2 steps per wave
    (3000, 16, 1, 128, 256, [3000, 1499, 2]),        # 16 heads per group, 1 step per wave
    (20000, 8, 2, 128, 4096, [20000, 16387, 4101]),  # 4 steps per wave
    (9000, 12, 1, 256, 4096, [8999, 600]),           # fewer kept blocks than places
])
def test_sparse_attn_decode(lmax, hq, hkv, d, budget, seq):
    bsz = len(seq)
    _say(f"decode attn seq={seq} heads={hq}/{hkv} d={d} K={budget}")
    q = _randn_bf16((bsz, hq, d), 31, 1 / math.sqrt(d))
    kc = _randn_bf16((bsz, lmax, hkv, d), 32, 1 / math.sqrt(d))
    vc = _randn_bf16((bsz, lmax, hkv, d), 33, 1 / math.sqrt(d))
    sel_np = np.concatenate([_random_selection([s - 1], budget // 4, 4, 40 + i) for i, s in enumerate(seq)])
    sl = torch.tensor(seq, dtype=torch.int32, device=DEV)
    out, lse = Q.qsa_sparse_attn_decode(q, kc, vc, sl, torch.from_numpy(sel_np).to(DEV))
    torch.cuda.synchronize()
    for b in range(bsz):
        t = seq[b] - 1
        toks = O.kept_tokens(sel_np[b], t, 4, t + 1)
        ref, ref_lse = O.attend(O.bf16_to_f64(bits(q[b])), O.bf16_to_f64(bits(kc[b][toks])),
                                O.bf16_to_f64(bits(vc[b][toks])), 1 / math.sqrt(d))
        compare_output(out[b], ref, f"decode b={b}")
        assert np.max(np.abs(lse[b].double().cpu().numpy() - ref_lse)) <= LSE_ABS


# ------------------------------------------------------------------------------------
# Whole path against the oracle's whole path
# ------------------------------------------------------------------------------------


class _Rows:
    """Host copy of selected rows of a large tensor, indexed by absolute row."""

    def __init__(self, shape, rows, data):
        self.shape = shape
        self._at = {int(r): j for j, r in enumerate(rows)}
        self._data = data

    def __getitem__(self, idx):
        if isinstance(idx, (int, np.integer)):
            return self._data[self._at[int(idx)]]
        return self._data[[self._at[int(i)] for i in idx]]


def _prefill_parity(name, rows=None, row_chunk=4096, n_aligned=64, max_inexact=2, **over):
    """The whole prefill path on the GPU against the oracle's whole path on `rows` (all
    rows by default), plus the first `n_aligned` needle-aligned rows (all of them when
    None) and the first and last rows. Selections must match (near-ties within the
    band are counted, at most max_inexact rows), outputs are compared with the oracle's
    attention over the GPU's own validated selection."""
    wl = workload(name, **over)
    _say(f"prefill {wl.name} lq={wl.lq} lk={wl.lk} q_pos0={wl.q_pos0} K={wl.budget} "
         f"row_chunk={row_chunk}")
    inp = generate(wl, device=DEV)
    out, lse, sel, kp = Q.qsa_prefill_forward(
        inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["w"], inp["k_idx"], budget=wl.budget,
        q_pos0=wl.q_pos0, k_pooled_prefix=inp["k_pooled_prefix"], row_chunk=row_chunk)
    torch.cuda.synchronize()
    if rows is None:
        rows = np.arange(wl.lq)
    al_rows, al_blocks = inp["aligned_rows"], inp["aligned_blocks"]
    if n_aligned is not None:
        al_rows, al_blocks = al_rows[:n_aligned], al_blocks[:n_aligned]
    rows = np.unique(np.concatenate([np.asarray(rows), al_rows, [0, wl.lq - 1]])).astype(np.int64)
    rows_t = torch.from_numpy(rows).to(DEV)

    def fetch(toks):
        tt = torch.from_numpy(toks).to(DEV)
        return (O.bf16_to_f64(bits(inp["k"][tt])), O.bf16_to_f64(bits(inp["v"][tt])))

    prefix = None if inp["k_pooled_prefix"] is None else bits(inp["k_pooled_prefix"])
    # Oracle end to end (its own pooling, scores, selection, attention) on the rows.
    qb = _Rows((wl.lq, wl.hq, wl.d), rows, bits(inp["q"][rows_t]))
    qib = bits(inp["q_idx"])
    w_np = inp["w"].cpu().numpy()
    res = O.forward_prefill(qb, None, None, qib, w_np, bits(inp["k_idx"]),
                            r=wl.r, budget=wl.budget, q_pos0=wl.q_pos0,
                            k_pooled_prefix_bits=prefix, rows=rows, n_keys=wl.lk,
                            fetch_kv=fetch, row_chunk=512)
    # Pooled keys: bit-exact.
    np.testing.assert_array_equal(bits(kp[wl.pooled_prefix_blocks:]), res["pooled"])
    kp_all = O.bf16_to_f64(bits(kp))
    own = (wl.q_pos0 + rows) // wl.r
    tol = score_abs_tol(O.bf16_to_f64(qib[rows]), w_np[rows], kp_all, own)
    sel_np = sel[rows_t].cpu().numpy()
    n_exact = 0
    for j, i in enumerate(rows):
        n_exact += check_selection_row(sel_np[j], res["scores"][j], int(own[j]), wl.n_sel,
                                       f"{wl.name} row {i}", abs_tol=tol[j])
    # Needle-aligned rows keep their needle.
    for i, b in zip(al_rows, al_blocks):
        j = int(np.searchsorted(rows, i))
        assert b in sel_np[j], f"row {i} lost needle block {b}"
    # Output: oracle attention on the GPU's own selection.
    ref = np.zeros((len(rows), wl.hq, wl.d))
    for j, i in enumerate(rows):
        t = wl.q_pos0 + int(i)
        toks = O.kept_tokens(sel_np[j], t, wl.r, wl.lk)
        kr, vr = fetch(toks)
        ref[j], _ = O.attend(O.bf16_to_f64(qb[i]), kr, vr, 1 / math.sqrt(wl.d))
    got = out[rows_t]
    max_abs, rel = compare_output(got, ref, wl.name)
    g64 = got.float().cpu().numpy().astype(np.float64)
    row_rel = (np.linalg.norm((g64 - ref).reshape(len(rows), -1), axis=1)
               / np.linalg.norm(ref.reshape(len(rows), -1), axis=1))
    _say(f"  rows={len(rows)} (aligned {len(al_rows)}) exact_sel={n_exact} "
         f"tie_band_rows={len(rows) - n_exact} max_abs={max_abs:.2e} rel_l2={rel:.2e} "
         f"row_rel_l2: worst={row_rel.max():.2e} p99={np.quantile(row_rel, 0.99):.2e} "
         f"(row {int(rows[np.argmax(row_rel)])})")
    assert len(rows) - n_exact <= max_inexact, f"{len(rows) - n_exact} rows in the tie band"
    return n_exact, len(rows)


def test_prefill_tiny_all_rows():
    _prefill_parity("tiny", n_aligned=None)


def test_prefill_tiny_small_chunks_ragged():
    # Row chunks that do not divide Lq, Lq not a multiple of the 64-row tile.
    _prefill_parity("tiny", row_chunk=300, lq=1001, lk=1001, n_aligned=None)


def test_prefill_generation_boundaries_against_oracle():
    # The attention runs in launches of one resident generation of workgroups. Rows on
    # both sides of those boundaries, a query window that starts past a pooled prefix,
    # ragged selection chunks.
    n = Q.qsa_sparse_attn_fwd_rows_per_launch(2, 256)
    _say(f"rows per attention launch: {n}")
    assert 2 <= n < 6000
    rows = sorted({0, 1, n - 1, n, n + 1, 2 * n - 1, 2 * n, 6001, 9999, 11999})
    _prefill_parity("prefill32k", rows=rows, row_chunk=2500, lq=12000, lk=40000, q_pos0=28000,
                    pooled_prefix_blocks=5000)


def test_attention_independent_of_row_split():
    # Each row's result depends on that row only: the attention over all rows equals,
    # bit for bit, the attention over arbitrary row slices (different launch splits).
    wl = workload("prefill32k", lq=6000, lk=40000, q_pos0=34000, pooled_prefix_blocks=5000)
    _say(f"attention row split lq={wl.lq} lk={wl.lk} q_pos0={wl.q_pos0}")
    inp = generate(wl, device=DEV)
    out, lse, sel, _ = Q.qsa_prefill_forward(
        inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["w"], inp["k_idx"], budget=wl.budget,
        q_pos0=wl.q_pos0, k_pooled_prefix=inp["k_pooled_prefix"], row_chunk=2500)
    o2 = torch.zeros_like(out)
    l2 = torch.zeros_like(lse)
    scale = 1.0 / math.sqrt(wl.d)
    for c0, c1 in ((0, 777), (777, 2000), (2000, 2001), (2001, 5999), (5999, 6000)):
        Q.qsa_sparse_attn_fwd(inp["q"][c0:c1], inp["k"], inp["v"], sel[c0:c1],
                              q_pos0=wl.q_pos0 + c0, scale=scale, out=o2[c0:c1], lse=l2[c0:c1])
    torch.cuda.synchronize()
    assert torch.equal(o2, out) and torch.equal(l2, lse)


# The full-size workloads in the selection chunks the benchmark uses (16384 rows):
# seeded random rows, needle-aligned rows (every one at 32K, 512 at 128K and on the
# 1M context) and the first and last rows; at most 1 row in 500 may sit in the tie band.

@pytest.mark.timeout(600)
def test_prefill_32k_sampled():
    rng = np.random.default_rng(21)
    rows = rng.choice(32768, 2048, replace=False)
    _prefill_parity("prefill32k", rows=rows, row_chunk=16384, n_aligned=None, max_inexact=10)


@pytest.mark.timeout(600)
def test_prefill_128k_sampled():
    rng = np.random.default_rng(22)
    rows = rng.choice(131072, 1536, replace=False)
    _prefill_parity("prefill128k", rows=rows, row_chunk=16384, n_aligned=512, max_inexact=4)


@pytest.mark.timeout(900)
def test_chunked_prefill_1m_sampled():
    rng = np.random.default_rng(23)
    rows = rng.choice(8192, 1536, replace=False)
    _prefill_parity("chunked1m", rows=rows, row_chunk=8192, n_aligned=512, max_inexact=4)


def test_decode_forward_mixed_lengths_and_fallback():
    # 4 sequences in a 160K-token cache (rows longer than one top-k workgroup):
    # full, ragged (not a multiple of r), short (everything fits in the budget) and
    # one whose two segments hold fewer candidates than places (the merge must select
    # over the whole row). Sequence 0's pooled keys grow along one direction that its
    # indexer queries share, so its best blocks are the last ones: the segment
    # candidates of the fused scan are truncated there and the merge must fall back
    # to the whole row.
    wl = workload("decode1m", batch=4, lk=163840)
    seq = [163840, 163840 - 4001, 1500, 5000]
    _say(f"decode forward mixed lengths {seq}")
    inp = generate(wl, device=DEV, seq_lens=seq)
    nblk = wl.lk // 4
    u = torch.nn.functional.normalize(torch.randn(wl.d_i, device=DEV), dim=0)
    ramp = torch.linspace(0.1, 1.0, nblk, device=DEV)
    inp["k_pooled"][0] = (ramp[:, None] * u[None, :]).to(torch.bfloat16)
    inp["q_idx"][0, 0] = u.to(torch.bfloat16)[None, :].expand(wl.h_i, -1)
    out, lse, sel = Q.qsa_decode_forward(inp["q"], inp["q_idx"], inp["w"], inp["k_pooled"],
                                         inp["k_cache"], inp["v_cache"], inp["seq_lens"],
                                         budget=wl.budget)
    torch.cuda.synchronize()

    def fetch(b, toks):
        tt = torch.from_numpy(toks).to(DEV)
        return (O.bf16_to_f64(bits(inp["k_cache"][b][tt])),
                O.bf16_to_f64(bits(inp["v_cache"][b][tt])))

    res = O.forward_decode(bits(inp["q"]), bits(inp["q_idx"])[:, 0], inp["w"].cpu().numpy()[:, 0],
                           bits(inp["k_pooled"]), np.array(seq), fetch, r=4, budget=wl.budget)
    sel_np = sel.cpu().numpy()
    for b in range(len(seq)):
        t = seq[b] - 1
        check_selection_row(sel_np[b], res["scores"][b], t // 4, wl.n_sel, f"decode b={b}",
                            abs_tol=_decode_tol(inp, b, t))
        toks = O.kept_tokens(sel_np[b], t, 4, t + 1)
        kr, vr = fetch(b, toks)
        ref, _ = O.attend(O.bf16_to_f64(bits(inp["q"][b])), kr, vr, 1 / math.sqrt(wl.d))
        compare_output(out[b], ref, f"decode b={b}")
    # the best blocks of sequence 0 are among its last ones (ties go to lower ids)
    assert sel_np[0][0] > (seq[0] - 1) // 4 - 4 * wl.n_sel


def test_decode_1m_full():
    wl = workload("decode1m")
    _say("decode1m: 8 x 1M")
    inp = generate(wl, device=DEV)
    out, lse, sel = Q.qsa_decode_forward(inp["q"], inp["q_idx"], inp["w"], inp["k_pooled"],
                                         inp["k_cache"], inp["v_cache"], inp["seq_lens"],
                                         budget=wl.budget)
    torch.cuda.synchronize()

    def fetch(b, toks):
        tt = torch.from_numpy(toks).to(DEV)
        return (O.bf16_to_f64(bits(inp["k_cache"][b][tt])),
                O.bf16_to_f64(bits(inp["v_cache"][b][tt])))

    kpb = bits(inp["k_pooled"])
    res = O.forward_decode(bits(inp["q"]), bits(inp["q_idx"])[:, 0], inp["w"].cpu().numpy()[:, 0],
                           kpb, inp["seq_lens"].cpu().numpy(), fetch, r=4, budget=wl.budget)
    sel_np = sel.cpu().numpy()
    for b in range(wl.batch):
        t = int(inp["seq_lens"][b]) - 1
        check_selection_row(sel_np[b], res["scores"][b], t // 4, wl.n_sel, f"decode b={b}",
                            abs_tol=_decode_tol(inp, b, t))
        toks = O.kept_tokens(sel_np[b], t, 4, t + 1)
        kr, vr = fetch(b, toks)
        ref, ref_lse = O.attend(O.bf16_to_f64(bits(inp["q"][b])), kr, vr, 1 / math.sqrt(wl.d))
        compare_output(out[b], ref, f"decode b={b}")
        assert np.max(np.abs(lse[b].double().cpu().numpy() - ref_lse)) <= LSE_ABS
