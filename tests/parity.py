"""Comparison rules between the HIP path and the oracle.

* Pooled keys: bit-exact.
* Selections: exact, except where the oracle's m-th and (m+1)-th ranked scores are
  within the band max(REL_GAP * |s_m|, abs_tol) of each other; there every id in the
  symmetric difference must have an oracle score within that band of s_m. abs_tol is
  the row's fp32 score error bound (score_abs_tol): it only matters where s_m is at or
  near 0 (rows whose ReLU leaves fewer than m positive scores), and it never lets a
  block whose score clearly exceeds the threshold be dropped. When both sides rank
  the very same fp32 scores (top-k tested alone) the rule is plain equality.
* Attention output (bf16): max-abs <= 2e-2 and relative L2 <= 5e-3 over the whole
  compared output, with the oracle run on the GPU's own (validated) selection.
* Attention gradients (fp32 outputs of the backward): relative L2 <= 1e-2 and max-abs
  <= 2e-2 * max |reference| per gradient. The GPU rounds each product's weight
  operand (P for dv, dS for dq and dk) to bf16 (relative 2^-9) and takes the row term
  D from the forward's bf16 output; two such roundings per gradient give twice the
  forward's 5e-3 rel-L2 budget.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import qsa_oracle as O

REL_GAP = 1e-3
SCORE_REL = 2e-5  # fp32 score error bound, relative to sum_h |w| * sum_c |q_c * k_c|
OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 5e-3
LSE_ABS = 2e-3
GRAD_REL_L2 = 1e-2
GRAD_MAX_REL = 2e-2


def score_abs_tol(q_idx: np.ndarray, w: np.ndarray, k_pooled: np.ndarray,
                  own: np.ndarray, chunk: int = 128) -> np.ndarray:
    """Per row, twice the largest fp32 error bound of its candidate scores:
    2 * SCORE_REL * max_{b < own} sum_h |w_h| * (|q_h| . |k_b|).

    q_idx [n, H_I, d_I], w [n, H_I], k_pooled [nblk, d_I] (fp64), own [n] block ids.
    Two scores' errors separate a pair that fp32 may rank the other way round."""
    n = q_idx.shape[0]
    out = np.zeros(n)
    ak = np.abs(k_pooled)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        tot = 0.0
        for h in range(q_idx.shape[1]):
            tot = tot + np.abs(w[c0:c1, h:h + 1]) * (np.abs(q_idx[c0:c1, h, :]) @ ak.T)
        cols = np.arange(k_pooled.shape[0])[None, :]
        tot = np.where(cols < np.asarray(own[c0:c1])[:, None], tot, 0.0)
        out[c0:c1] = 2.0 * SCORE_REL * tot.max(axis=1) if tot.shape[1] else 0.0
    return out


def check_selection_row(sel_gpu: np.ndarray, scores_ref: np.ndarray, own: int, n_sel: int,
                        where: str = "", abs_tol: float = 0.0) -> bool:
    """Validate one GPU selection row against the oracle's scores of that row.

    Returns True when it equals the oracle's selection, False when it differs only
    inside the tolerated near-tie band; raises AssertionError otherwise.
    """
    sel_gpu = np.asarray(sel_gpu, dtype=np.int64)
    kept = sel_gpu[sel_gpu >= 0]
    n_valid = min(n_sel, own + 1)
    assert len(kept) == n_valid, f"{where}: {len(kept)} kept, expected {n_valid}"
    assert np.all(sel_gpu[n_valid:] == -1), f"{where}: bad padding"
    assert kept[-1] == own, f"{where}: own block {own} not last ({kept[-1]})"
    assert np.all(np.diff(kept) > 0), f"{where}: not strictly ascending"
    ref = O.select_blocks(scores_ref, own, n_sel)
    if np.array_equal(ref, sel_gpu):
        return True
    gap = O.ranked_threshold_gap(scores_ref, own, n_sel)
    assert gap is not None, f"{where}: mismatch although every block fits"
    s_m, s_m1 = gap
    band = max(REL_GAP * abs(s_m), float(abs_tol))
    assert (s_m - s_m1) <= band, \
        f"{where}: selection differs with a clear gap ({s_m} vs {s_m1}, band {band})"
    diff = np.setxor1d(ref[ref >= 0], kept)
    for b in diff:
        assert abs(scores_ref[b] - s_m) <= band, \
            f"{where}: block {b} (score {scores_ref[b]}) outside the tie band of {s_m} ({band})"
    return False


def compare_output(out_gpu: torch.Tensor, out_ref: np.ndarray, where: str = ""):
    got = out_gpu.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - out_ref)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - out_ref) / max(np.linalg.norm(out_ref), 1e-300))
    assert max_abs <= OUT_MAX_ABS, f"{where}: max-abs {max_abs:.3e} > {OUT_MAX_ABS}"
    assert rel <= OUT_REL_L2, f"{where}: rel-L2 {rel:.3e} > {OUT_REL_L2}"
    return max_abs, rel


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def compare_grad(got_gpu: torch.Tensor, ref: np.ndarray, where: str = ""):
    got = got_gpu.double().cpu().numpy()
    scale = max(float(np.abs(ref).max()), 1e-300)
    max_rel = float(np.abs(got - ref).max()) / scale if ref.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    assert rel <= GRAD_REL_L2, f"{where}: rel-L2 {rel:.3e} > {GRAD_REL_L2}"
    assert max_rel <= GRAD_MAX_REL, f"{where}: max-abs / max|ref| {max_rel:.3e} > {GRAD_MAX_REL}"
    return max_rel, rel
