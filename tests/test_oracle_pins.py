"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test checks the oracle against a library routine, a brute-force or closed-form
result, a hand-derived fixture, or an invariant the method's definition fixes, so
that a dropped term, a wrong sign or index, or a transposed operand fails one of
them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import qsa_oracle as O
from synth import bf16_bits, generate, generate_varlen, workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x: np.ndarray) -> np.ndarray:
    """bf16 bits of fp32-exact values via torch's own conversion (library routine)."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return bf16_bits(t)


# ------------------------------------------------------------------------------------
# bf16 encoding
# ------------------------------------------------------------------------------------


def test_bf16_round_trip_and_torch_agreement():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-39, -1e-40]]).astype(np.float32)
    ref = bf16_bits(torch.from_numpy(x).to(torch.bfloat16))  # fp32 -> bf16, RNE
    mine = O.f64_to_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(mine, ref)
    np.testing.assert_array_equal(O.f64_to_bf16(O.bf16_to_f64(ref)), ref)


def test_bf16_halfway_cases_round_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: even significand (1.0) wins.
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: even (1+2^-6) wins.
    vals = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -40])
    got = O.bf16_to_f64(O.f64_to_bf16(vals))
    np.testing.assert_array_equal(got, [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7])
    # A value that double rounding through fp32 would get wrong: just above halfway by
    # less than fp32 resolution.
    v = np.array([1 + 2.0 ** -8 + 2.0 ** -30])
    assert O.bf16_to_f64(O.f64_to_bf16(v))[0] == 1 + 2.0 ** -7


# ------------------------------------------------------------------------------------
# Pooling
# ------------------------------------------------------------------------------------


def test_pool_matches_torch_mean_and_drops_partial_block():
    rng = np.random.default_rng(1)
    k = _bits(rng.standard_normal((4 * 37 + 3, 16)) / 8)
    pooled = O.pool_keys(k, 4)
    assert pooled.shape == (37, 16)
    kt = torch.from_numpy(O.bf16_to_f64(k)).view(-1)[: 37 * 4 * 16].view(37, 4, 16)
    mean = kt.mean(dim=1)  # fp64 mean; exact in fp32 for these magnitudes
    assert torch.equal(mean.float().double(), mean)
    np.testing.assert_array_equal(pooled, bf16_bits(mean.float().to(torch.bfloat16)))


def test_pool_of_identical_keys_is_exact():
    u = _bits(np.array([[0.3, -1.25, 7.0, 1e-3]]))
    k = np.repeat(u, 4, axis=0)
    np.testing.assert_array_equal(O.pool_keys(k, 4), u)


# ------------------------------------------------------------------------------------
# Hand-derived selections (tests/golden/hand_selection.json)
# ------------------------------------------------------------------------------------


def _hand_pooled(kind: str) -> np.ndarray:
    kp = np.zeros((16, 4))
    for b in range(16):
        if kind == "one_hot":
            kp[b, b % 4] = (b + 1) if b % 2 == 0 else -(b + 1)
        else:
            kp[b] = [1.0, 0.0, 0.0, 0.0] if b == 2 else [b / 64, 1.0, 1.0, 1.0]
    return kp


def _hand_cases():
    with open(os.path.join(GOLDEN, "hand_selection.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        for row in case["rows"]:
            yield case["pooled_keys"], row


@pytest.mark.parametrize("kind,row", list(_hand_cases()))
def test_hand_built_selection(kind, row):
    kp = _hand_pooled(kind)
    k_idx = _bits(np.repeat(kp, 4, axis=0))  # every token of a block holds its pooled key
    pooled = O.pool_keys(k_idx, 4)
    np.testing.assert_array_equal(O.bf16_to_f64(pooled), kp)
    t = row["t"]
    s = O.index_scores(np.array(row["q"], float)[None, None, :], np.array([[row["w"]]]),
                       O.bf16_to_f64(pooled), np.array([t]), 4)[0]
    sel = O.select_blocks(s[: t // 4], t // 4, 4)
    assert sel.tolist() == row["sel"], row["why"]


# ------------------------------------------------------------------------------------
# Full coverage: QSA equals dense causal attention when the budget covers the prefix
# ------------------------------------------------------------------------------------


def _dense_causal_bruteforce(q, k, v, scale):
    """Dense causal attention written as masked matrices (not the oracle's gather)."""
    lq, hq, d = q.shape
    grp = hq // k.shape[1]
    out = np.zeros_like(q)
    lse = np.zeros((lq, hq))
    mask = np.tril(np.ones((lq, lq), bool))
    for h in range(hq):
        z = scale * q[:, h, :] @ k[:, h // grp, :].T
        z = np.where(mask, z, -np.inf)
        mx = z.max(axis=1, keepdims=True)
        e = np.exp(z - mx)
        out[:, h, :] = e @ v[:, h // grp, :] / e.sum(axis=1, keepdims=True)
        lse[:, h] = (mx + np.log(e.sum(axis=1, keepdims=True)))[:, 0]
    return out, lse


def _small_prefill(L=256, hq=4, hkv=2, d=32, budget=256, seed=5):
    wl = workload("tiny", lq=L, lk=L, hq=hq, hkv=hkv, d=d, d_i=16, budget=budget, seed=seed,
                  needle_spacing=64)
    return wl, generate(wl)


def _run_oracle(wl, inp, **kw):
    return O.forward_prefill(bf16_bits(inp["q"]), bf16_bits(inp["k"]), bf16_bits(inp["v"]),
                             bf16_bits(inp["q_idx"]), inp["w"].numpy(), bf16_bits(inp["k_idx"]),
                             r=wl.r, budget=wl.budget, q_pos0=wl.q_pos0,
                             k_pooled_prefix_bits=(None if inp["k_pooled_prefix"] is None
                                                   else bf16_bits(inp["k_pooled_prefix"])), **kw)


def test_full_budget_equals_dense_causal_attention():
    wl, inp = _small_prefill(L=256, budget=256)
    res = _run_oracle(wl, inp)
    q, k, v = (O.bf16_to_f64(bf16_bits(inp[n])) for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(wl.d)
    ref, ref_lse = _dense_causal_bruteforce(q, k, v, scale)
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["lse"], ref_lse, rtol=0, atol=1e-12)
    # The textbook routine: torch's scaled_dot_product_attention, fp64 on the CPU.
    tq = torch.from_numpy(q).permute(1, 0, 2)
    grp = wl.hq // wl.hkv
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(grp, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(grp, dim=0)
    sdpa = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                            scale=scale)
    np.testing.assert_allclose(res["out"], sdpa.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_rows_before_budget_are_dense():
    wl, inp = _small_prefill(L=512, budget=128)  # n_sel = 32: rows t < 128 keep everything
    res = _run_oracle(wl, inp, rows=np.arange(0, 128, 7))
    q, k, v = (O.bf16_to_f64(bf16_bits(inp[n])) for n in ("q", "k", "v"))
    ref, _ = _dense_causal_bruteforce(q[:128], k[:128], v[:128], 1.0 / math.sqrt(wl.d))
    np.testing.assert_allclose(res["out"], ref[res["rows"]], rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------
# Invariants of every selection row, and library reductions
# ------------------------------------------------------------------------------------


def test_selection_invariants_and_bruteforce_ranking():
    wl = workload("tiny")
    inp = generate(wl)
    rows = np.concatenate([np.arange(0, 2048, 37), inp["aligned_rows"][:40], [2047]])
    res = _run_oracle(wl, inp, rows=rows)
    n_sel = wl.n_sel
    for j, i in enumerate(res["rows"]):
        t = int(i)
        own = t // 4
        sel = res["sel"][j]
        kept = sel[sel >= 0]
        assert len(kept) == min(n_sel, own + 1)
        assert kept[-1] == own and np.all(np.diff(kept) > 0) and kept.max() <= own
        assert np.all(sel[len(kept):] == -1)
        s = res["scores"][j]
        # Brute force: plain Python sort by (score desc, id asc).
        m = min(n_sel - 1, own)
        best = sorted(range(own), key=lambda b: (-s[b], b))[:m]
        assert sorted(best) == kept[:-1].tolist()
        if m < own:
            unsel = np.setdiff1d(np.arange(own), kept)
            assert s[kept[:-1]].min() >= s[unsel].max()
    for i, b in zip(inp["aligned_rows"][:40], inp["aligned_blocks"][:40]):
        j = int(np.nonzero(res["rows"] == i)[0][0])
        assert b in res["sel"][j], "needle-aligned row lost its needle"


def test_scores_reduce_to_one_gemv_when_relu_is_identity():
    rng = np.random.default_rng(3)
    q = np.abs(rng.standard_normal((9, 4, 16)))
    kp = np.abs(rng.standard_normal((30, 16)))
    pos = np.full(9, 4 * 30 + 3)
    s = O.index_scores(q, np.ones((9, 4)), kp, pos, 4)
    np.testing.assert_allclose(s, np.einsum("nc,bc->nb", q.sum(axis=1), kp), rtol=1e-13)


def test_scores_with_relu_against_explicit_loops():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 4, 8))
    w = rng.random((3, 4))
    kp = rng.standard_normal((10, 8))
    pos = np.array([7, 20, 43])
    s = O.index_scores(q, w, kp, pos, 4)
    for n in range(3):
        for b in range(10):
            if b >= pos[n] // 4:
                assert np.isnan(s[n, b])
                continue
            tot = 0.0
            for h in range(4):
                dot = sum(q[n, h, c] * kp[b, c] for c in range(8))
                tot += w[n, h] * (dot if dot > 0 else 0.0)
            assert abs(s[n, b] - tot) < 1e-12


def test_metamorphic_weight_scale_and_head_permutation():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 4, 16))
    w = rng.random((4, 4))
    kp = rng.standard_normal((200, 16))
    pos = np.array([400, 500, 801, 803])
    s = O.index_scores(q, w, kp, pos, 4)
    s3 = O.index_scores(q, 3.5 * w, kp, pos, 4)
    perm = [2, 0, 3, 1]
    sp = O.index_scores(q[:, perm], w[:, perm], kp, pos, 4)
    np.testing.assert_allclose(sp, s, rtol=1e-13)
    for n in range(4):
        own = pos[n] // 4
        a = O.select_blocks(s[n, :own], own, 32)
        b = O.select_blocks(s3[n, :own], own, 32)
        np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------------------------------
# Closed forms of the attention stage
# ------------------------------------------------------------------------------------


def test_attention_closed_forms():
    rng = np.random.default_rng(6)
    n, hq, hkv, d = 40, 6, 2, 16
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((n, hkv, d))
    # Constant V per group -> output is that constant.
    v = np.zeros((n, hkv, d))
    v[:, 0, :] = 1.5
    v[:, 1, :] = -2.0
    o, _ = O.attend(q, k, v, 0.3)
    np.testing.assert_allclose(o[:3], 1.5, rtol=1e-14)
    np.testing.assert_allclose(o[3:], -2.0, rtol=1e-14)
    # q = 0 -> uniform weights: output is the mean of the rows, lse = log(n).
    v = rng.standard_normal((n, hkv, d))
    o, lse = O.attend(np.zeros((hq, d)), k, v, 0.3)
    np.testing.assert_allclose(o[:3], np.broadcast_to(v[:, 0].mean(0), (3, d)), rtol=1e-12)
    np.testing.assert_allclose(o[3:], np.broadcast_to(v[:, 1].mean(0), (3, d)), rtol=1e-12)
    np.testing.assert_allclose(lse, math.log(n), rtol=1e-14)
    # One dominant logit (+40 over the others) -> output is that key's value.
    k = np.zeros((n, hkv, d))
    q = np.zeros((hq, d))
    q[:, 0] = 1.0
    k[17, :, 0] = 40.0
    o, lse = O.attend(q, k, v, 1.0)
    np.testing.assert_allclose(o[:3], np.broadcast_to(v[17, 0], (3, d)), atol=1e-15)
    np.testing.assert_allclose(lse, 40.0 + math.log1p((n - 1) * math.exp(-40)), rtol=1e-15)


def test_own_block_masks_future_keys():
    # Query at t = 4*b + 1 reads only tokens 4b and 4b+1 of its own block.
    sel = np.array([0, 3, 5, -1])
    toks = O.kept_tokens(sel, 21, 4, 64)
    assert toks.tolist() == [0, 1, 2, 3, 12, 13, 14, 15, 20, 21]


# ------------------------------------------------------------------------------------
# Decode = last prefill row; chunked prefill = rows of the full prefill
# ------------------------------------------------------------------------------------


def test_decode_equals_prefill_last_row():
    L = 640
    wl, inp = _small_prefill(L=L, budget=64, seed=8)
    res = _run_oracle(wl, inp, rows=[L - 1, L - 2])
    pooled = O.pool_keys(bf16_bits(inp["k_idx"]), 4)
    kb, vb = bf16_bits(inp["k"]), bf16_bits(inp["v"])

    def fetch(b, toks):
        return O.bf16_to_f64(kb[toks]), O.bf16_to_f64(vb[toks])

    qb = bf16_bits(inp["q"])
    qib = bf16_bits(inp["q_idx"])
    w = inp["w"].numpy()
    for j, seqlen in enumerate([L, L - 1]):
        row = seqlen - 1
        dec = O.forward_decode(qb[row][None], qib[row][None], w[row][None], pooled[None],
                               [seqlen], fetch, r=4, budget=64)
        np.testing.assert_array_equal(dec["sel"][0], res["sel"][j])
        np.testing.assert_allclose(dec["out"][0], res["out"][j], rtol=0, atol=1e-13)


def test_chunked_prefill_equals_full_prefill_rows():
    L, prefix = 768, 512
    wl, inp = _small_prefill(L=L, budget=64, seed=9)
    full = _run_oracle(wl, inp, rows=np.arange(prefix, L, 5))
    kb = bf16_bits(inp["k_idx"])
    pooled_prefix = O.pool_keys(kb[:prefix], 4)
    chunk = O.forward_prefill(bf16_bits(inp["q"])[prefix:], bf16_bits(inp["k"]),
                              bf16_bits(inp["v"]), bf16_bits(inp["q_idx"])[prefix:],
                              inp["w"].numpy()[prefix:], kb[prefix:], r=4, budget=64,
                              q_pos0=prefix, k_pooled_prefix_bits=pooled_prefix,
                              rows=np.arange(0, L - prefix, 5))
    np.testing.assert_array_equal(chunk["sel"], full["sel"])
    np.testing.assert_allclose(chunk["out"], full["out"], rtol=0, atol=1e-13)


# ------------------------------------------------------------------------------------
# Positional encoding of the pooled keys
# ------------------------------------------------------------------------------------


def _torch_rope_complex(x: np.ndarray, pos: np.ndarray, rope_dim: int, theta: float):
    """The same rotation written as complex multiplication (torch, fp64)."""
    h = rope_dim // 2
    t = torch.from_numpy(np.array(x, dtype=np.float64))
    inv = torch.tensor(float(theta), dtype=torch.float64) ** (
        -2.0 * torch.arange(h, dtype=torch.float64) / rope_dim)
    ang = torch.from_numpy(np.asarray(pos, dtype=np.float64))[:, None] * inv[None, :]
    z = torch.complex(t[:, :h], t[:, h:rope_dim]) * torch.polar(torch.ones_like(ang), ang)
    out = t.clone()
    out[:, :h], out[:, h:rope_dim] = z.real, z.imag
    return out.numpy()


@pytest.mark.parametrize("rope_dim,first_block", [(16, 0), (64, 7), (128, 1000)])
def test_pooled_encoding_against_torch_complex_rotation(rope_dim, first_block):
    rng = np.random.default_rng(rope_dim)
    k = _bits(rng.standard_normal((4 * 300 + 3, 128)) / math.sqrt(128))
    got = O.pool_keys(k, 4, (rope_dim, 1e4), first_block=first_block)
    mean = torch.from_numpy(O.bf16_to_f64(k)[:1200]).reshape(300, 4, 128).mean(dim=1).numpy()
    ref = _torch_rope_complex(mean, (first_block + np.arange(300)) * 4, rope_dim, 1e4)
    np.testing.assert_array_equal(got, O.f64_to_bf16(ref))
    # columns past rope_dim are the plain mean; position 0 is the identity
    np.testing.assert_array_equal(got[:, rope_dim:], O.pool_keys(k, 4)[:, rope_dim:])
    if first_block == 0:
        np.testing.assert_array_equal(got[0], O.pool_keys(k, 4)[0])


def test_rotary_scores_depend_on_offset_only():
    # Rotating the query at t and the key at p keeps norms and gives a dot product that
    # depends on t - p only (shifting both by 1000 changes nothing), for every pair.
    rng = np.random.default_rng(11)
    q, k = rng.standard_normal((50, 64)), rng.standard_normal((50, 64))
    t, p = rng.integers(0, 5000, 50), rng.integers(0, 5000, 50)
    for rd in (16, 64):
        qr, kr = O.rope_rotate(q, t, rd, 1e6), O.rope_rotate(k, p, rd, 1e6)
        qs, ks = O.rope_rotate(q, t + 1000, rd, 1e6), O.rope_rotate(k, p + 1000, rd, 1e6)
        np.testing.assert_allclose((qr * kr).sum(1), (qs * ks).sum(1), rtol=1e-9, atol=1e-9)
        np.testing.assert_allclose(np.linalg.norm(qr, axis=1), np.linalg.norm(q, axis=1),
                                   rtol=1e-12)
    np.testing.assert_array_equal(O.rope_rotate(q, t, 0, 1e4), q)


def test_encoded_chunked_prefill_equals_full_prefill_rows():
    # With the encoding, a prefix pooled earlier (its blocks at their own positions) and
    # the chunk's new blocks pooled from first_block on give the full prefill's rows.
    L, prefix, pe = 768, 512, (16, 1e4)
    wl, inp = _small_prefill(L=L, budget=64, seed=9)
    full = _run_oracle(wl, inp, rows=np.arange(prefix, L, 5), pe=pe)
    kb = bf16_bits(inp["k_idx"])
    pooled_prefix = O.pool_keys(kb[:prefix], 4, pe)
    chunk = O.forward_prefill(bf16_bits(inp["q"])[prefix:], bf16_bits(inp["k"]),
                              bf16_bits(inp["v"]), bf16_bits(inp["q_idx"])[prefix:],
                              inp["w"].numpy()[prefix:], kb[prefix:], r=4, budget=64,
                              q_pos0=prefix, k_pooled_prefix_bits=pooled_prefix,
                              rows=np.arange(0, L - prefix, 5), pe=pe)
    np.testing.assert_array_equal(chunk["sel"], full["sel"])
    np.testing.assert_allclose(chunk["out"], full["out"], rtol=0, atol=1e-13)
    plain = _run_oracle(wl, inp, rows=np.arange(prefix, L, 5))
    assert not np.array_equal(plain["sel"], full["sel"])  # the encoding changes selections


# ------------------------------------------------------------------------------------
# Packed variable-length batches
# ------------------------------------------------------------------------------------


def _varlen_oracle(inp, budget, **kw):
    return O.forward_prefill_varlen(
        bf16_bits(inp["q"]), bf16_bits(inp["k"]), bf16_bits(inp["v"]), bf16_bits(inp["q_idx"]),
        inp["w"].numpy(), bf16_bits(inp["k_idx"]), inp["cu_q"].numpy(), inp["cu_k"].numpy(),
        r=4, budget=budget, **kw)


def test_varlen_full_budget_equals_dense_attention_per_sequence():
    # Budget above every length: each sequence is dense attention over its own keys,
    # queries aligned to its last tokens (a prefix packed in for the second one).
    lens = [(37, 37), (20, 53), (65, 65), (1, 6)]
    wl = workload("tiny", hq=4, hkv=2, d=16, d_i=16, budget=256, seed=3, needle_spacing=0)
    inp = generate_varlen(wl, lens)
    res = _varlen_oracle(inp, 256)
    q, k, v = (torch.from_numpy(O.bf16_to_f64(bf16_bits(inp[n]))) for n in ("q", "k", "v"))
    cq, ck = inp["cu_q"].numpy(), inp["cu_k"].numpy()
    scale = 1.0 / math.sqrt(wl.d)
    for b, (lq, lk) in enumerate(lens):
        qs = q[cq[b]:cq[b + 1]].permute(1, 0, 2)
        ks = k[ck[b]:ck[b + 1]].permute(1, 0, 2).repeat_interleave(2, dim=0)
        vs = v[ck[b]:ck[b + 1]].permute(1, 0, 2).repeat_interleave(2, dim=0)
        allow = torch.arange(lk)[None, :] <= (lk - lq + torch.arange(lq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=allow,
                                                               scale=scale)
        logits = torch.where(allow, scale * qs @ ks.transpose(1, 2), -torch.inf)
        np.testing.assert_allclose(res["out"][cq[b]:cq[b + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose(res["lse"][cq[b]:cq[b + 1]],
                                   torch.logsumexp(logits, -1).T.numpy(), rtol=0, atol=1e-12)


def test_varlen_sequences_are_isolated_and_rows_valid():
    # Under a budget (selection active), changing every input of sequence 0 leaves the
    # other sequences' results bit-identical; every row's selection is a valid one of
    # its own sequence (local ids, own block, size, order).
    lens = [(40, 40), (24, 64), (33, 33)]
    wl = workload("tiny", hq=4, hkv=2, d=16, d_i=16, budget=16, seed=4, needle_spacing=0)
    inp = generate_varlen(wl, lens)
    res = _varlen_oracle(inp, 16)
    alt = dict(inp)
    g = torch.Generator().manual_seed(99)
    for n in ("q", "k", "v", "q_idx", "k_idx"):
        t = inp[n].clone()
        end = int(inp["cu_q" if n in ("q", "q_idx") else "cu_k"][1])
        t[:end] = torch.randn(t[:end].shape, generator=g).to(t.dtype)
        alt[n] = t
    res2 = _varlen_oracle(alt, 16)
    first = int(inp["cu_q"][1])
    assert not np.array_equal(res["out"][:first], res2["out"][:first])
    np.testing.assert_array_equal(res["sel"][first:], res2["sel"][first:])
    np.testing.assert_array_equal(res["out"][first:], res2["out"][first:])
    cq = inp["cu_q"].numpy()
    for b, (lq, lk) in enumerate(lens):
        for i in range(lq):
            t = lk - lq + i
            own = t // 4
            row = res["sel"][cq[b] + i]
            kept = row[row >= 0]
            assert len(kept) == min(4, own + 1) and kept[-1] == own
            assert np.all(np.diff(kept) > 0) and np.all(row[len(kept):] == -1)


def test_paged_fetcher_matches_contiguous_cache():
    # Scatter a contiguous cache into randomly ordered pages (spare pages hold noise):
    # the paged fetcher returns the contiguous rows, and decode through it is identical.
    rng = np.random.default_rng(8)
    bsz, lmax, hkv, d, P = 3, 96, 2, 8, 16
    kc = _bits(rng.standard_normal((bsz, lmax, hkv, d)))
    vc = _bits(rng.standard_normal((bsz, lmax, hkv, d)))
    n_pages = bsz * lmax // P + 5
    perm = rng.permutation(n_pages)[: bsz * lmax // P].reshape(bsz, lmax // P)
    kp_pool = _bits(rng.standard_normal((n_pages * P, hkv, d)))
    vp_pool = _bits(rng.standard_normal((n_pages * P, hkv, d)))
    for b in range(bsz):
        for p in range(lmax // P):
            kp_pool[perm[b, p] * P:(perm[b, p] + 1) * P] = kc[b, p * P:(p + 1) * P]
            vp_pool[perm[b, p] * P:(perm[b, p] + 1) * P] = vc[b, p * P:(p + 1) * P]
    fetch = O.paged_fetcher(kp_pool, vp_pool, perm, P)
    toks = rng.choice(lmax, 40, replace=False)
    for b in range(bsz):
        kr, vr = fetch(b, toks)
        np.testing.assert_array_equal(kr, O.bf16_to_f64(kc[b, toks]))
        np.testing.assert_array_equal(vr, O.bf16_to_f64(vc[b, toks]))
    q = _bits(rng.standard_normal((bsz, 4, d)))
    qi = _bits(rng.standard_normal((bsz, 2, 8)))
    w = rng.uniform(size=(bsz, 2))
    kpool = _bits(rng.standard_normal((bsz, lmax // 4, 8)))
    lens = np.array([96, 61, 7])
    ref = O.forward_decode(q, qi, w, kpool, lens,
                           lambda b, t: (O.bf16_to_f64(kc[b, t]), O.bf16_to_f64(vc[b, t])),
                           r=4, budget=32)
    got = O.forward_decode(q, qi, w, kpool, lens, fetch, r=4, budget=32)
    np.testing.assert_array_equal(got["sel"], ref["sel"])
    np.testing.assert_array_equal(got["out"], ref["out"])


# ------------------------------------------------------------------------------------
# Backward of the sparse attention over a fixed selection
# ------------------------------------------------------------------------------------


def _bwd_case(seed, lq=12, lk=24, hq=4, hkv=2, d=8, r=4, n_sel=3, q_pos0=12, qscale=1.0):
    rng = np.random.default_rng(seed)
    q = _bits(rng.standard_normal((lq, hq, d)) * qscale)
    k = _bits(rng.standard_normal((lk, hkv, d)))
    v = _bits(rng.standard_normal((lk, hkv, d)))
    sel = np.full((lq, n_sel), -1, dtype=np.int64)
    for i in range(lq):
        own = (q_pos0 + i) // r
        others = rng.choice(own, min(n_sel - 1, own), replace=False) if own else []
        row = np.sort(np.concatenate([np.asarray(others, dtype=np.int64), [own]]))
        sel[i, : len(row)] = row
    dout = rng.standard_normal((lq, hq, d))
    return q, k, v, sel, dout


def _loss(q, k, v, sel, dout, r, q_pos0, scale):
    """sum(dout * o) as a function of fp64 q, k, v (the oracle's forward)."""
    tot = 0.0
    for i in range(q.shape[0]):
        toks = O.kept_tokens(sel[i], q_pos0 + i, r, k.shape[0])
        o, _ = O.attend(q[i], k[toks], v[toks], scale)
        tot += float((dout[i] * o).sum())
    return tot


def test_backward_matches_central_differences():
    # The analytic gradients against numerical derivatives of the oracle's own forward
    # (a dropped softmax-Jacobian term, a wrong sign or a transposed operand fails).
    q, k, v, sel, dout = _bwd_case(30)
    r, q_pos0, scale = 4, 12, 0.7
    g = O.backward_prefill(q, k, v, sel, dout, r=r, q_pos0=q_pos0, scale=scale)
    qf, kf, vf = O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v)
    eps = 1e-6
    rng = np.random.default_rng(31)
    for name, arr, grad in (("q", qf, g["dq"]), ("k", kf, g["dk"]), ("v", vf, g["dv"])):
        for _ in range(25):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args = {"q": qf, "k": kf, "v": vf}
            args[name] = plus
            lp = _loss(args["q"], args["k"], args["v"], sel, dout, r, q_pos0, scale)
            args[name] = minus
            lm = _loss(args["q"], args["k"], args["v"], sel, dout, r, q_pos0, scale)
            num = (lp - lm) / (2 * eps)
            assert abs(num - grad[idx]) <= 1e-7 * max(1.0, abs(num)), (name, idx, num, grad[idx])


def test_backward_matches_torch_autograd_dense_masked():
    # Library routine: torch autograd (CPU, fp64) through a dense softmax attention whose
    # mask allows exactly each row's kept tokens.
    q, k, v, sel, dout = _bwd_case(32, lq=10, lk=20, hq=6, hkv=2, d=16, n_sel=3, q_pos0=8)
    r, q_pos0, scale = 4, 8, 0.25
    g = O.backward_prefill(q, k, v, sel, dout, r=r, q_pos0=q_pos0, scale=scale)
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    mask = torch.zeros((lq, lk), dtype=torch.bool)
    for i in range(lq):
        mask[i, torch.from_numpy(O.kept_tokens(sel[i], q_pos0 + i, r, lk))] = True
    qt = torch.from_numpy(O.bf16_to_f64(q)).requires_grad_()
    kt = torch.from_numpy(O.bf16_to_f64(k)).requires_grad_()
    vt = torch.from_numpy(O.bf16_to_f64(v)).requires_grad_()
    grp = hq // hkv
    kk = kt.repeat_interleave(grp, dim=1)  # [lk, hq, d], head h reads group h // grp
    vv = vt.repeat_interleave(grp, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.transpose(0, 1), kk.transpose(0, 1), vv.transpose(0, 1),
        attn_mask=mask[None], scale=scale).transpose(0, 1)
    (o * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(g["dq"], qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dk"], kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dv"], vt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_closed_forms_and_invariants():
    r, q_pos0, scale = 4, 12, 0.5
    q, k, v, sel, dout = _bwd_case(33)
    lk = k.shape[0]
    # (1) Softmax rows sum to one, so the logits' gradient sums to zero per (row, head):
    #     the key gradients of a KV group sum to zero over all keys.
    g = O.backward_prefill(q, k, v, sel, dout, r=r, q_pos0=q_pos0, scale=scale)
    np.testing.assert_allclose(g["dk"].sum(axis=0), 0.0, atol=1e-12)
    # (2) dv sums dout over the reading rows with weight p: summed over keys it is the
    #     sum of every row's dout per group (p sums to one).
    grp = q.shape[1] // k.shape[1]
    want = dout.reshape(dout.shape[0], k.shape[1], grp, -1).sum(axis=(0, 2))
    np.testing.assert_allclose(g["dv"].sum(axis=0), want, atol=1e-10)
    # (3) V constant per group: o does not depend on q or k, so dq = dk = 0.
    vc = np.repeat(v[:1], lk, axis=0)
    g = O.backward_prefill(q, k, vc, sel, dout, r=r, q_pos0=q_pos0, scale=scale)
    np.testing.assert_allclose(g["dq"], 0.0, atol=1e-12)
    np.testing.assert_allclose(g["dk"], 0.0, atol=1e-12)
    # (4) q = 0: uniform weights over each row's kept tokens, so dv[j] is the sum of
    #     dout / |J_i| over the rows i that read j.
    qz = np.zeros_like(q)
    g = O.backward_prefill(qz, k, v, sel, dout, r=r, q_pos0=q_pos0, scale=scale)
    want = np.zeros_like(g["dv"])
    for i in range(q.shape[0]):
        toks = O.kept_tokens(sel[i], q_pos0 + i, r, lk)
        for h in range(q.shape[1]):
            want[toks, h // grp] += dout[i, h] / len(toks)
    np.testing.assert_allclose(g["dv"], want, atol=1e-12)


# ------------------------------------------------------------------------------------
# Indexer warm-up: KL distillation target, loss and the indexer's gradients
# ------------------------------------------------------------------------------------


def test_kl_target_against_torch_softmax_and_max_pool():
    # Library routines: torch softmax over the causal logits, summed over heads, then
    # torch's max_pool1d over r-token windows, normalised.
    rng = np.random.default_rng(50)
    hq, hkv, d, r = 6, 2, 16, 4
    k = O.bf16_to_f64(_bits(rng.standard_normal((40, hkv, d))))
    for t in (3, 4, 17, 39):
        q = O.bf16_to_f64(_bits(rng.standard_normal((hq, d))))
        got = O.kl_block_target(q, k[: t + 1], t, r, 0.3)
        kk = torch.from_numpy(k[: t + 1]).repeat_interleave(hq // hkv, dim=1)  # [t+1, hq, d]
        z = 0.3 * torch.einsum("hd,jhd->hj", torch.from_numpy(q), kk)
        a = torch.softmax(z, dim=1).sum(0)
        own = t // r
        if own == 0:
            assert got.size == 0
            continue
        pooled = torch.nn.functional.max_pool1d(a[None, None, : own * r], r, r)[0, 0]
        np.testing.assert_allclose(got, (pooled / pooled.sum()).numpy(), rtol=1e-12, atol=0)


def test_kl_target_closed_forms():
    rng = np.random.default_rng(51)
    hq, hkv, d, r, t = 4, 1, 8, 4, 23
    k = rng.standard_normal((t + 1, hkv, d))
    # q = 0: uniform attention, so every complete block pools the same value.
    np.testing.assert_allclose(O.kl_block_target(np.zeros((hq, d)), k, t, r, 1.0),
                               np.full(t // r, 1.0 / (t // r)), rtol=1e-14)
    # One key dominating every head: the target sits on its block.
    q = np.zeros((hq, d))
    q[:, 0] = 1.0
    k2 = k.copy()
    k2[:, :, 0] = 0.0
    k2[9, :, 0] = 80.0
    p = O.kl_block_target(q, k2, t, r, 1.0)
    assert p.argmax() == 9 // r and p[9 // r] > 0.99


def test_indexer_kl_against_torch_kl_div_and_autograd():
    rng = np.random.default_rng(52)
    s = rng.standard_normal(37) * 3
    p = rng.random(37)
    p[[3, 10]] = 0.0
    p /= p.sum()
    loss, ds = O.indexer_kl(s, p)
    st = torch.from_numpy(s).requires_grad_()
    ref = torch.nn.functional.kl_div(torch.log_softmax(st, 0), torch.from_numpy(p),
                                     reduction="sum")
    ref.backward()
    ref_v = float(ref.detach())
    assert abs(loss - ref_v) <= 1e-12 * max(1.0, abs(ref_v))
    np.testing.assert_allclose(ds, st.grad.numpy(), rtol=1e-12, atol=1e-15)
    # KL is zero exactly when the target is the indexer's own distribution.
    q = np.exp(s - s.max())
    q /= q.sum()
    assert abs(O.indexer_kl(s, q)[0]) < 1e-13


def test_index_scores_backward_central_differences():
    # d/dx of sum(ds * s(x)) numerically, for q_idx, w and the pooled keys (inputs drawn
    # so that no q.k sits within the step of the ReLU's kink).
    rng = np.random.default_rng(53)
    n, hh, di, nblk, r = 5, 3, 6, 7, 4
    pos = np.array([4, 9, 17, 28, 31])
    q = rng.standard_normal((n, hh, di))
    w = rng.random((n, hh))
    kp = rng.standard_normal((nblk, di))
    ds = rng.standard_normal((n, nblk))
    dq, dw, dkp = O.index_scores_backward(q, w, kp, ds, pos, r)

    def f(q_, w_, kp_):
        sc = O.index_scores(q_, w_, kp_, pos, r)
        return float(np.nansum(sc * ds))

    eps = 1e-6
    for name, arr, grad in (("q", q, dq), ("w", w, dw), ("kp", kp, dkp)):
        for idx in np.ndindex(arr.shape):
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args = {"q": q, "w": w, "kp": kp}
            args[name] = plus
            fp = f(args["q"], args["w"], args["kp"])
            args[name] = minus
            fm = f(args["q"], args["w"], args["kp"])
            num = (fp - fm) / (2 * eps)
            assert abs(num - grad[idx]) <= 1e-7 * max(1.0, abs(num)), (name, idx, num, grad[idx])


def test_pool_keys_backward_against_autograd():
    # The mean pooling's gradient, per token: torch's avg_pool1d (windows of r, stride
    # r, a partial tail window dropped) differentiated by autograd in fp64. Every token
    # of a complete block gets its block's gradient / r; the tail tokens get 0.
    rng = np.random.default_rng(54)
    assert np.all(O.pool_keys_backward(np.zeros((0, 4)), 4, 3) == 0)  # no complete block
    for n_tokens, di, nblk in ((4 * 7 + 2, 6, 7), (4 * 5, 3, 5), (4 + 3, 4, 1)):
        dkp = rng.standard_normal((nblk, di))
        x = torch.from_numpy(rng.standard_normal((n_tokens, di))).requires_grad_()
        pooled = torch.nn.functional.avg_pool1d(x.T[None], kernel_size=4, stride=4)[0].T
        assert pooled.shape == (nblk, di)
        (pooled * torch.from_numpy(dkp)).sum().backward()
        got = O.pool_keys_backward(dkp, 4, n_tokens)
        assert got.shape == (n_tokens, di)
        np.testing.assert_allclose(got, x.grad.numpy(), rtol=1e-15, atol=0)


def test_ranked_threshold_gap_hand_cases():
    # Candidates ranked by score: 5, 3, 3, 1, 0.5 (blocks 0..4; the entries after the
    # own block are not candidates). With n_sel places the row keeps m = n_sel - 1
    # earlier blocks: the m-th and (m+1)-th ranked scores, written out by hand.
    s = np.array([3.0, 5.0, 0.5, 3.0, 1.0, 99.0, 99.0])
    own = 5
    assert O.ranked_threshold_gap(s, own, 3) == (3.0, 3.0)   # m = 2: 5, [3], 3
    assert O.ranked_threshold_gap(s, own, 4) == (3.0, 1.0)   # m = 3: 5, 3, [3], 1
    assert O.ranked_threshold_gap(s, own, 5) == (1.0, 0.5)   # m = 4
    assert O.ranked_threshold_gap(s, own, 2) == (5.0, 3.0)   # m = 1
    assert O.ranked_threshold_gap(s, own, 6) is None         # m = 5: every candidate kept
    assert O.ranked_threshold_gap(s, own, 40) is None
    assert O.ranked_threshold_gap(s, own, 1) is None         # only the own block
    assert O.ranked_threshold_gap(s, 0, 3) is None           # no candidate
    # ReLU zeros and a signed zero: 2, 0, -0, 0 -> m = 2 gives (0, 0)
    z = np.array([0.0, 2.0, -0.0, 0.0])
    assert O.ranked_threshold_gap(z, 4, 3) == (0.0, 0.0)
    assert O.ranked_threshold_gap(z, 4, 2) == (2.0, 0.0)


def test_ranked_threshold_gap_brute_force():
    # Against the brute-force ranking of select_blocks' own rule on random rows with
    # ties: the m-th kept block's score and the best dropped block's score.
    rng = np.random.default_rng(55)
    for _ in range(200):
        own = int(rng.integers(1, 40))
        n_sel = int(rng.integers(1, 45))
        s = rng.integers(0, 6, size=own + 3).astype(np.float64)
        ranked = sorted(range(own), key=lambda b: (-s[b], b))
        m = min(n_sel - 1, own)
        want = None if (m == 0 or m >= own) else (s[ranked[m - 1]], s[ranked[m]])
        assert O.ranked_threshold_gap(s, own, n_sel) == want
