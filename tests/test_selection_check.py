"""CPU checks of the selection-parity rule the GPU tests apply (near-tie
branch included): a set that trades a clearly better channel for a worse one
is rejected, valid top-k sets within the gap are accepted."""
import numpy as np
import pytest

from tests.gpu_helpers import GAP, check_scores, check_selection


def _scores():
    # k = 4: the 4th and 5th scores are within the gap, the top three are not
    s = np.array([9.0, 1.0, 5.0, 3.0, 3.0 * (1 - GAP / 4), 0.5, 7.0, 0.1])
    return s[None, :]


def test_near_tie_accepts_either_tied_channel():
    s = _scores()
    assert check_selection(np.array([[0, 2, 3, 6]]), s, 4) == 0
    assert check_selection(np.array([[0, 2, 4, 6]]), s, 4) == 0


def test_near_tie_rejects_dropping_the_top_channel():
    s = _scores()
    # the top channel (0) swapped for the (k+1)-th (4): every chosen score is
    # still >= s_{k+1}, so only the must-include rule can catch it
    with pytest.raises(AssertionError, match="not chosen"):
        check_selection(np.array([[2, 3, 4, 6]]), s, 4)


def test_near_tie_rejects_a_low_channel():
    s = _scores()
    with pytest.raises(AssertionError):
        check_selection(np.array([[0, 1, 2, 6]]), s, 4)


def test_exact_branch_and_structure():
    s = np.array([[4.0, 3.0, 2.0, 1.0]])
    assert check_selection(np.array([[0, 1]]), s, 2) == 1
    with pytest.raises(AssertionError):
        check_selection(np.array([[0, 2]]), s, 2)
    with pytest.raises(AssertionError):
        check_selection(np.array([[1, 0]]), s, 2)          # not ascending
    with pytest.raises(AssertionError):
        check_selection(np.array([[1, 1]]), s, 2)          # not distinct


def test_score_closeness():
    ref = np.array([[1.0, 2.0, 4.0]])
    check_scores(ref * (1 + 5e-5), ref, 1e-4)
    with pytest.raises(AssertionError):
        check_scores(ref * (1 + 5e-4), ref, 1e-4)
