"""CPU oracle of the Qwen Sparse Attention (QSA) forward path, of the sparse
attention's backward over a fixed selection, and of the indexer's KL warm-up loss.

TEST INFRASTRUCTURE ONLY. This is the plain, slow, obviously correct fp64 numpy
statement of what the path computes, used to check the HIP library. Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
product path never calls it. It shares no code with the HIP library.

Sources (the pages describing QSA; cited by title and section):

* [DR] "On the Design of Qwen3.8-Next Architecture" (summary page), section
  "four architecture components", item 2 "Qwen Sparse Attention (QSA)": the
  indexer scores micro-blocks of r=4 tokens; keys are first mean-pooled, then a
  positional encoding is added; the indexer has 4 MQA query heads; the token
  budget is K=2048; the route follows DeepSeek DSA's light indexer + top-k.
* [MR] "Qwen3.8-Flash-Next" (Miles RL recipe page), section 1 "Model
  Introduction": each full-attention layer projects its own indexer queries and
  compressed keys, scores them, keeps ``indexer_budget`` key tokens per query and
  attention reads only those; 24 heads, 2 query groups, kv-channels 256.
* [RA] Release article "Qwen3.8-Flash-Next开源", section "GDN+QSA": the light
  indexer aggregates the sequence into micro-blocks, rates importance per block,
  then attends only over the most relevant regions.

Readings where the pages leave a step open (each is stated where it is used):

* Score (DSA reading): s[t,b] = sum_h w[t,h] * max(0, qI[t,h] . kbar[b]); no extra
  global scale (a positive scale cannot change a ranking).
* Pooling is the mean over the r keys of a complete block, rounded once to bf16;
  a trailing partial block is never pooled. The positional encoding [DR] adds after
  pooling is optional: a partial rotary encoding of the pooled key at its block's
  first-token position (``rope_rotate``; the pages give no form).
* Only complete blocks strictly before the query's own block b(t) = t // r are
  scored; the own block is always kept and counts toward the budget, so
  n_sel = K // r blocks are kept in all. Ties go to the lower block index; -0.0
  equals +0.0. With fewer causal blocks than n_sel - 1 every block is kept.
* One selection per query token, shared by all heads; head h uses KV group
  h // (Hq // Hkv). Inside the kept blocks, keys after the query are masked.
* lse is the natural-log sum of exp of the scaled logits.

Parity pins: every function here is checked against something other than itself
in tests/test_oracle_pins.py (library routines, brute force, closed forms,
hand-derived selections in tests/golden/).
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------------------
# bf16 encoding (inputs arrive as raw bf16 bit patterns, uint16)
# --------------------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode raw bf16 bit patterns: a bf16 value is the top half of an IEEE fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (round to nearest, ties to even), return bit patterns.

    bf16 keeps 8 significant bits and fp32's exponent range; its spacing in
    [2^e', 2^(e'+1)) is 2^(e'-7), and 2^-133 below the smallest normal 2^-126.
    The rounding is done once, directly from fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)  # x = m * 2**e with 0.5 <= |m| < 1
    q_exp = np.maximum(e - 8, -133)  # exponent of the bf16 spacing at x
    y = np.ldexp(np.rint(np.ldexp(x, -q_exp)), q_exp)  # rint: ties to even
    return (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------------------
# Stage 1: micro-block mean pooling of the indexer keys  [DR]
# --------------------------------------------------------------------------------------


def rope_rotate(x: np.ndarray, pos: np.ndarray, rope_dim: int, theta: float) -> np.ndarray:
    """Rotary encoding of rows x [n, d] at positions pos [n] (fp64), half-split form:
    for i < h = rope_dim / 2 the pair (x[i], x[i + h]) turns by pos * theta^(-2i/rope_dim);
    columns from rope_dim on are unchanged. (Reading of [DR]'s unnamed positional
    encoding: the partial rotary encoding of the model's attention.)"""
    y = np.array(x, dtype=np.float64, copy=True)
    if rope_dim == 0:
        return y
    h = rope_dim // 2
    inv = np.power(float(theta), -2.0 * np.arange(h, dtype=np.float64) / rope_dim)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = y[:, :h].copy(), y[:, h:rope_dim].copy()
    y[:, :h] = a * c - b * s
    y[:, h:rope_dim] = b * c + a * s
    return y


def pool_keys(k_idx_bits: np.ndarray, r: int, pe=None, first_block: int = 0) -> np.ndarray:
    """Mean-pool r consecutive indexer keys per complete block, rounded to bf16 [DR].

    k_idx_bits: [n_tokens, d_I] bf16 bits. Returns [n_tokens // r, d_I] bf16 bits.
    With pe = (rope_dim, theta) the mean is first encoded at the block's position
    (first_block + b) * r, the position of its first token ([DR]: keys are pooled
    first, then the position is encoded); mean and rotation in fp64, one rounding.
    """
    x = bf16_to_f64(k_idx_bits)
    nb = x.shape[0] // r
    blocks = x[: nb * r].reshape(nb, r, x.shape[1])
    m = blocks.sum(axis=1) / r
    if pe is not None and pe[0]:
        m = rope_rotate(m, (first_block + np.arange(nb)) * r, int(pe[0]), float(pe[1]))
    return f64_to_bf16(m)


# --------------------------------------------------------------------------------------
# Stage 2: light MQA indexer scores at block granularity  [DR], [RA]
# --------------------------------------------------------------------------------------


def index_scores(q_idx: np.ndarray, w: np.ndarray, k_pooled: np.ndarray,
                 positions: np.ndarray, r: int) -> np.ndarray:
    """Block scores for query rows at absolute ``positions``.

    q_idx [n, H_I, d_I] and w [n, H_I] as fp64, k_pooled [nblk, d_I] fp64.
    Returns [n, nblk] fp64 with s[i, b] = sum_h w[i,h] * max(0, q_idx[i,h] . k_pooled[b])
    for b < positions[i] // r, and NaN where the block is not scored.
    """
    n, n_heads, _ = q_idx.shape
    s = np.zeros((n, k_pooled.shape[0]), dtype=np.float64)
    for h in range(n_heads):
        dots = q_idx[:, h, :] @ k_pooled.T  # one plain matmul per indexer head
        s += w[:, h : h + 1] * np.maximum(dots, 0.0)
    own = np.asarray(positions) // r
    cols = np.arange(k_pooled.shape[0])
    s[cols[None, :] >= own[:, None]] = np.nan
    return s


# --------------------------------------------------------------------------------------
# Stage 3: block top-k under the token budget  [MR], [DR]
# --------------------------------------------------------------------------------------


def select_blocks(scores_row: np.ndarray, own_block: int, n_sel: int) -> np.ndarray:
    """Kept blocks of one query row: ascending block ids, padded with -1.

    scores_row holds the scores of blocks 0..own_block-1. The own block is always
    kept; of the earlier blocks the n_sel - 1 best are kept, ranked by score
    (descending) then block id (ascending).
    """
    cand = np.asarray(scores_row[:own_block], dtype=np.float64)
    m = min(n_sel - 1, own_block)
    ids = np.arange(own_block)
    order = np.lexsort((ids, -cand))  # primary key: -score ascending; then id ascending
    sel = np.full(n_sel, -1, dtype=np.int64)
    sel[:m] = np.sort(order[:m])
    sel[m] = own_block
    return sel


def ranked_threshold_gap(scores_row: np.ndarray, own_block: int, n_sel: int):
    """(m-th best score, (m+1)-th best score) of the candidates, or None if all are kept."""
    cand = np.asarray(scores_row[:own_block], dtype=np.float64)
    m = min(n_sel - 1, own_block)
    if m >= own_block or m == 0:
        return None
    srt = np.sort(cand)[::-1]
    return float(srt[m - 1]), float(srt[m])


# --------------------------------------------------------------------------------------
# Stage 4: exact softmax attention over the kept tokens  [MR]
# --------------------------------------------------------------------------------------


def kept_tokens(sel_row: np.ndarray, t: int, r: int, n_keys: int) -> np.ndarray:
    """Token ids read by query position t: every token of a kept block, j <= t."""
    blocks = np.asarray(sel_row)[np.asarray(sel_row) >= 0]
    toks = (blocks[:, None] * r + np.arange(r)[None, :]).reshape(-1)
    return toks[(toks <= t) & (toks < n_keys)]


def attend(q_t: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float):
    """Softmax attention of one query token over given key/value rows.

    q_t [Hq, d], k_rows/v_rows [n, Hkv, d] fp64; head h reads KV group h // (Hq//Hkv).
    Returns (o [Hq, d], lse [Hq]), lse the natural-log normaliser of the scaled logits.
    """
    hq, d = q_t.shape
    hkv = k_rows.shape[1]
    grp = hq // hkv
    o = np.zeros((hq, d), dtype=np.float64)
    lse = np.zeros(hq, dtype=np.float64)
    for h in range(hq):
        g = h // grp
        z = scale * (k_rows[:, g, :] @ q_t[h])
        mx = z.max()
        p = np.exp(z - mx)
        den = p.sum()
        o[h] = (p @ v_rows[:, g, :]) / den
        lse[h] = mx + np.log(den)
    return o, lse


def attend_backward(q_t: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                    do_t: np.ndarray, scale: float):
    """Gradients of attend(q_t, k_rows, v_rows) given do_t [Hq, d], the gradient of
    the loss with respect to the output o [Hq, d].

    The selection is a constant of the backward pass ([MR] ships a forward and a
    backward sparse-attention kernel over selection rows built outside the kernel):
    no gradient reaches the indexer through the top-k. Per head h (KV group g), with
    z = scale * K_g q_h, p = softmax(z), o_h = p V_g:
      dv_g += p (outer) do_h,    dp = V_g do_h,
      dz = p * (dp - p . dp)     (softmax Jacobian),
      dq_h = scale * dz K_g,     dk_g += scale * dz (outer) q_h.
    Returns (dq [Hq, d], dk [n, Hkv, d], dv [n, Hkv, d]).
    """
    hq, d = q_t.shape
    n, hkv, _ = k_rows.shape
    grp = hq // hkv
    dq = np.zeros((hq, d), dtype=np.float64)
    dk = np.zeros((n, hkv, d), dtype=np.float64)
    dv = np.zeros((n, hkv, d), dtype=np.float64)
    for h in range(hq):
        g = h // grp
        z = scale * (k_rows[:, g, :] @ q_t[h])
        p = np.exp(z - z.max())
        p /= p.sum()
        dv[:, g, :] += np.outer(p, do_t[h])
        dp = v_rows[:, g, :] @ do_t[h]
        dz = p * (dp - p @ dp)
        dq[h] = scale * (dz @ k_rows[:, g, :])
        dk[:, g, :] += scale * np.outer(dz, q_t[h])
    return dq, dk, dv


def backward_prefill(q_bits, k_bits, v_bits, sel, dout, *, r: int, q_pos0: int = 0,
                     scale: Optional[float] = None) -> dict:
    """Backward of the sparse attention over given selections, for every query row.

    q_bits [Lq, Hq, d], k_bits/v_bits [Lk, Hkv, d] (bf16 bit patterns); sel [Lq, n_sel]
    block ids (-1 padded); dout [Lq, Hq, d] fp64 (the output gradient). Row i is at
    position q_pos0 + i and reads kept_tokens(sel[i]). The key and value gradients
    sum the contributions of every row that read the token.
    Returns dq [Lq, Hq, d], dk and dv [Lk, Hkv, d], fp64.
    """
    lq, hq, d = q_bits.shape
    lk, hkv, _ = k_bits.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    k = bf16_to_f64(k_bits)
    v = bf16_to_f64(v_bits)
    dq = np.zeros((lq, hq, d), dtype=np.float64)
    dk = np.zeros((lk, hkv, d), dtype=np.float64)
    dv = np.zeros((lk, hkv, d), dtype=np.float64)
    for i in range(lq):
        toks = kept_tokens(sel[i], q_pos0 + i, r, lk)
        dq[i], dkr, dvr = attend_backward(bf16_to_f64(q_bits[i]), k[toks], v[toks],
                                          np.asarray(dout[i], dtype=np.float64), scale)
        np.add.at(dk, toks, dkr)
        np.add.at(dv, toks, dvr)
    return {"dq": dq, "dk": dk, "dv": dv}


# --------------------------------------------------------------------------------------
# Indexer warm-up: KL distillation of the full attention onto the block scores  [DR]
# --------------------------------------------------------------------------------------
# [DR] trains the indexer in two stages, the first a warm-up that distils the full
# attention distribution, max-pooled to the block level, into the indexer by a KL
# loss. Readings: the heads' probabilities are summed (one indexer serves all heads),
# the target lives on the blocks the indexer scores (complete blocks before the own
# block, which is always kept) and is L1-normalised there; the indexer's distribution
# is the softmax of its scores over the same blocks; the loss is KL(target || indexer)
# summed over query rows; the target carries no gradient.


def kl_block_target(q_t: np.ndarray, k_rows: np.ndarray, t: int, r: int, scale: float):
    """Distillation target of the query at position t over blocks 0 .. t // r - 1.

    q_t [Hq, d]; k_rows [t + 1, Hkv, d] holds keys 0..t (fp64). The full causal
    attention probabilities of every head are summed, max-pooled over each block's r
    tokens and normalised to sum to one. Empty when no block is scored.
    """
    own = t // r
    if own == 0:
        return np.zeros(0)
    hq = q_t.shape[0]
    grp = hq // k_rows.shape[1]
    a = np.zeros(t + 1, dtype=np.float64)
    for h in range(hq):
        z = scale * (k_rows[:, h // grp, :] @ q_t[h])
        e = np.exp(z - z.max())
        a += e / e.sum()
    pooled = a[: own * r].reshape(own, r).max(axis=1)
    return pooled / pooled.sum()


def indexer_kl(scores_row: np.ndarray, target: np.ndarray):
    """KL(target || softmax(scores)) over one row's scored blocks, and its gradient with
    respect to the scores, softmax(scores) - target. Returns (loss, ds)."""
    if len(scores_row) == 0:
        return 0.0, np.zeros(0)
    m = scores_row.max()
    lse = m + np.log(np.exp(scores_row - m).sum())
    logq = scores_row - lse
    nz = target > 0  # 0 * log 0 = 0
    loss = float(np.sum(target[nz] * (np.log(target[nz]) - logq[nz])))
    return loss, np.exp(logq) - target


def index_scores_backward(q_idx: np.ndarray, w: np.ndarray, k_pooled: np.ndarray,
                          ds: np.ndarray, positions: np.ndarray, r: int):
    """Gradients of the block scores (index_scores) with respect to q_idx [n, H_I, d_I],
    w [n, H_I] and k_pooled [nblk, d_I], given ds [n, nblk] = dL/ds (entries of blocks a
    row does not score are ignored). With z = q_idx[i,h] . k_pooled[b]:
      dw[i,h] = sum_b ds[i,b] max(0, z),  dz = ds[i,b] w[i,h] [z > 0],
      dq_idx[i,h] = sum_b dz k_pooled[b],  dk_pooled[b] = sum_{i,h} dz q_idx[i,h].
    The ReLU's derivative at 0 is taken as 0. Returns (dq_idx, dw, dk_pooled).
    """
    n, n_heads, _ = q_idx.shape
    own = np.asarray(positions) // r
    cols = np.arange(k_pooled.shape[0])
    g = np.where(cols[None, :] < own[:, None], np.nan_to_num(ds), 0.0)
    dq = np.zeros_like(q_idx, dtype=np.float64)
    dw = np.zeros((n, n_heads), dtype=np.float64)
    dkp = np.zeros_like(k_pooled, dtype=np.float64)
    for h in range(n_heads):
        z = q_idx[:, h, :] @ k_pooled.T
        dw[:, h] = (g * np.maximum(z, 0.0)).sum(axis=1)
        dz = g * w[:, h : h + 1] * (z > 0)
        dq[:, h, :] = dz @ k_pooled
        dkp += dz.T @ q_idx[:, h, :]
    return dq, dw, dkp


def pool_keys_backward(dk_pooled: np.ndarray, r: int, n_tokens: int) -> np.ndarray:
    """Gradient of the mean pooling: each token of a complete block gets its block's
    gradient / r (the bf16 rounding of the pooled key is passed straight through);
    tokens of a trailing partial block get 0."""
    out = np.zeros((n_tokens, dk_pooled.shape[1]), dtype=np.float64)
    nb = min(dk_pooled.shape[0], n_tokens // r)
    out[: nb * r] = np.repeat(dk_pooled[:nb] / r, r, axis=0)
    return out


# --------------------------------------------------------------------------------------
# Whole path
# --------------------------------------------------------------------------------------


def _rows_fetcher(k_bits: np.ndarray, v_bits: np.ndarray):
    def fetch(tokens: np.ndarray):
        return bf16_to_f64(k_bits[tokens]), bf16_to_f64(v_bits[tokens])
    return fetch


def forward_prefill(q_bits, k_bits, v_bits, q_idx_bits, w, k_idx_bits, *, r: int, budget: int,
                    q_pos0: int = 0, scale: Optional[float] = None,
                    k_pooled_prefix_bits: Optional[np.ndarray] = None,
                    rows: Optional[Sequence[int]] = None, n_keys: Optional[int] = None,
                    fetch_kv: Optional[Callable] = None, row_chunk: int = 2048,
                    pe=None) -> dict:
    """QSA prefill for query rows ``rows`` (default: all).

    q_bits [Lq, Hq, d]; k_bits/v_bits [Lk, Hkv, d] (or ``fetch_kv(tokens)`` returning
    fp64 rows, with ``n_keys`` = Lk); q_idx_bits [Lq, H_I, d_I]; w [Lq, H_I];
    k_idx_bits holds the raw indexer keys of the tokens after the pooled prefix
    (k_pooled_prefix_bits, [P, d_I], or none). Query row i is at position q_pos0 + i.
    Returns the pooled keys of the new blocks, and per row: scores, selection,
    output and lse. pe = (rope_dim, theta) encodes the new pooled keys (see pool_keys).
    """
    lq, hq, d = q_bits.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    n_sel = budget // r
    if fetch_kv is None:
        fetch_kv = _rows_fetcher(k_bits, v_bits)
        n_keys = k_bits.shape[0]
    n_prefix = 0 if k_pooled_prefix_bits is None else len(k_pooled_prefix_bits)
    pooled_new = pool_keys(k_idx_bits, r, pe, first_block=n_prefix)
    if k_pooled_prefix_bits is not None and len(k_pooled_prefix_bits):
        pooled_all = np.concatenate([k_pooled_prefix_bits, pooled_new], axis=0)
    else:
        pooled_all = pooled_new
    kp = bf16_to_f64(pooled_all)
    rows = np.arange(lq) if rows is None else np.asarray(rows, dtype=np.int64)
    wq = np.asarray(w, dtype=np.float64)
    sels = np.zeros((len(rows), n_sel), dtype=np.int64)
    outs = np.zeros((len(rows), hq, d), dtype=np.float64)
    lses = np.zeros((len(rows), hq), dtype=np.float64)
    score_rows = []
    for c0 in range(0, len(rows), row_chunk):
        rr = rows[c0 : c0 + row_chunk]
        pos = q_pos0 + rr
        s = index_scores(bf16_to_f64(q_idx_bits[rr]), wq[rr], kp, pos, r)
        for j, (i, t) in enumerate(zip(rr, pos)):
            own = int(t) // r
            score_rows.append(s[j, :own].copy())
            sel = select_blocks(s[j, :own], own, n_sel)
            toks = kept_tokens(sel, int(t), r, n_keys)
            k_rows, v_rows = fetch_kv(toks)
            o, lse = attend(bf16_to_f64(q_bits[i]), k_rows, v_rows, scale)
            sels[c0 + j], outs[c0 + j], lses[c0 + j] = sel, o, lse
    return {"pooled": pooled_new, "rows": rows, "scores": score_rows, "sel": sels,
            "out": outs, "lse": lses}


def forward_prefill_varlen(q_bits, k_bits, v_bits, q_idx_bits, w, k_idx_bits, cu_q, cu_k, *,
                           r: int, budget: int, scale: Optional[float] = None,
                           rows: Optional[Sequence[int]] = None, pe=None) -> dict:
    """QSA prefill of a packed batch ([MR] section 5.3 "Rollout & SGLang": packed THD
    tensors). Sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 and key tokens
    cu_k[b] .. cu_k[b+1]-1; its queries are its last tokens (row i of the sequence
    at position lk_b - lq_b + i). Each sequence is an independent prefill: its blocks,
    scores, selection (ids local to the sequence) and attention see only its own keys.
    ``rows`` are packed query rows (default all). Returns the pooled keys of each
    sequence and, per requested row in order: scores, selection, output and lse.
    """
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    total_q = int(cu_q[-1])
    rows = np.arange(total_q) if rows is None else np.asarray(rows, dtype=np.int64)
    seq_of = np.searchsorted(cu_q, rows, side="right") - 1
    hq, d = q_bits.shape[1:]
    n_sel = budget // r
    out = {"pooled": [], "scores": [None] * len(rows), "sel": np.zeros((len(rows), n_sel), np.int64),
           "out": np.zeros((len(rows), hq, d)), "lse": np.zeros((len(rows), hq))}
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        mine = np.nonzero(seq_of == b)[0]
        res = forward_prefill(q_bits[q0:q1], k_bits[k0:k1], v_bits[k0:k1], q_idx_bits[q0:q1],
                              np.asarray(w)[q0:q1], k_idx_bits[k0:k1], r=r, budget=budget,
                              q_pos0=int((k1 - k0) - (q1 - q0)), scale=scale,
                              rows=rows[mine] - q0, pe=pe)
        out["pooled"].append(res["pooled"])
        for j, m in enumerate(mine):
            out["scores"][m] = res["scores"][j]
            out["sel"][m], out["out"][m], out["lse"][m] = res["sel"][j], res["out"][j], res["lse"][j]
    return out


def paged_fetcher(k_pool_bits, v_pool_bits, block_table, page_size: int):
    """``fetch_kv(b, tokens)`` for a paged K/V cache: token j of sequence b sits at pool
    slot block_table[b][j // page_size] * page_size + j % page_size (pools
    [n_slots, Hkv, d] of raw bf16 bits)."""
    table = np.asarray(block_table, dtype=np.int64)

    def fetch(b: int, tokens: np.ndarray):
        tokens = np.asarray(tokens, dtype=np.int64)
        slots = table[b, tokens // page_size] * page_size + tokens % page_size
        return bf16_to_f64(k_pool_bits[slots]), bf16_to_f64(v_pool_bits[slots])
    return fetch


def forward_decode(q_bits, q_idx_bits, w, k_pooled_bits, seq_lens, fetch_kv, *, r: int,
                   budget: int, scale: Optional[float] = None) -> dict:
    """QSA decode: one new query token per sequence, at position seq_lens[b] - 1.

    q_bits [B, Hq, d]; q_idx_bits [B, H_I, d_I]; w [B, H_I]; k_pooled_bits
    [B, nblk, d_I] (the pooled-key cache); ``fetch_kv(b, tokens)`` returns fp64
    K and V rows [n, Hkv, d] of sequence b. Returns per sequence: scores,
    selection, output and lse.
    """
    bsz, hq, d = q_bits.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    n_sel = budget // r
    sels = np.zeros((bsz, n_sel), dtype=np.int64)
    outs = np.zeros((bsz, hq, d), dtype=np.float64)
    lses = np.zeros((bsz, hq), dtype=np.float64)
    score_rows = []
    for b in range(bsz):
        t = int(seq_lens[b]) - 1
        own = t // r
        kp = bf16_to_f64(k_pooled_bits[b, :own])
        s = index_scores(bf16_to_f64(q_idx_bits[b])[None], np.asarray(w[b], np.float64)[None],
                         kp, np.array([t]), r)[0] if own else np.zeros(0)
        score_rows.append(s[:own].copy())
        sel = select_blocks(s[:own], own, n_sel)
        toks = kept_tokens(sel, t, r, t + 1)
        k_rows, v_rows = fetch_kv(b, toks)
        outs[b], lses[b] = attend(bf16_to_f64(q_bits[b]), k_rows, v_rows, scale)
        sels[b] = sel
    return {"scores": score_rows, "sel": sels, "out": outs, "lse": lses}
