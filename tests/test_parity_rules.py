"""The comparison rules of tests/parity.py, exercised on hand-made rows (CPU only):
a selection that drops a clearly better block must be rejected, whatever the score
at the threshold; swaps inside the tie band are accepted and counted as inexact."""
import numpy as np
import pytest

from parity import REL_GAP, check_selection_row, score_abs_tol


def test_zero_threshold_does_not_waive_a_dropped_block():
    # Scores [5, 0, 0, 0, 0], own block 5, 3 places (2 earlier blocks): the oracle
    # keeps blocks 0 and 1. A row keeping 1 and 2 drops the block scoring 5.0.
    s = np.array([5.0, 0.0, 0.0, 0.0, 0.0])
    with pytest.raises(AssertionError):
        check_selection_row(np.array([1, 2, 5]), s, 5, 3)
    # even with a generous fp32 error floor the 5.0 block may not go
    with pytest.raises(AssertionError):
        check_selection_row(np.array([1, 2, 5]), s, 5, 3, abs_tol=1e-3)
    assert check_selection_row(np.array([0, 1, 5]), s, 5, 3) is True


def test_swaps_among_exact_zeros_are_tolerated():
    # Blocks scoring exactly 0 are tied; fp32 may turn one of them into a tiny
    # positive score and keep it first.
    s = np.array([3.0, 0.0, 0.0, 0.0, 0.0])
    assert check_selection_row(np.array([0, 3, 5]), s, 5, 3) is False


def test_near_tie_band():
    s = np.array([5.0, 1.0, 1.0 - 0.5 * REL_GAP, 0.2])
    assert check_selection_row(np.array([0, 1, 4]), s, 4, 3) is True
    assert check_selection_row(np.array([0, 2, 4]), s, 4, 3) is False
    s2 = np.array([5.0, 1.0, 1.0 - 10 * REL_GAP, 0.2])
    with pytest.raises(AssertionError):
        check_selection_row(np.array([0, 2, 4]), s2, 4, 3)


def test_absolute_floor_near_zero():
    # The oracle keeps block 2 (score 1e-9) over the zero blocks; an fp32 score of 0
    # for it makes the GPU keep block 1. Only an absolute floor (the row's fp32 error
    # bound) tolerates that; the relative band of 1e-12 does not.
    s = np.array([3.0, 0.0, 1e-9, 0.0])
    with pytest.raises(AssertionError):
        check_selection_row(np.array([0, 1, 4]), s, 4, 3)
    assert check_selection_row(np.array([0, 1, 4]), s, 4, 3, abs_tol=1e-6) is False


def test_structure_is_checked():
    s = np.array([3.0, 2.0, 1.0, 0.5])
    with pytest.raises(AssertionError):      # own block missing
        check_selection_row(np.array([0, 1, 2]), s, 4, 3)
    with pytest.raises(AssertionError):      # not ascending
        check_selection_row(np.array([1, 0, 4]), s, 4, 3)
    with pytest.raises(AssertionError):      # wrong count
        check_selection_row(np.array([0, 4, -1]), s, 4, 3)


def test_score_abs_tol_is_the_largest_candidate_bound():
    # one head, w = 2; |q| . |k_b| = 1, 3, 10 for the three pooled keys; row 0 owns
    # block 2 (candidates 0 and 1), row 1 owns block 3 (all three)
    q = np.array([[[1.0, -1.0]], [[1.0, -1.0]]])
    w = np.array([[2.0], [-2.0]])
    kp = np.array([[0.5, 0.5], [-1.0, 2.0], [5.0, -5.0]])
    tol = score_abs_tol(q, w, kp, np.array([2, 3]))
    np.testing.assert_allclose(tol, [2 * 2e-5 * 2 * 3, 2 * 2e-5 * 2 * 10])
