"""The routing near-tie rule of the parity tests (tests/oracle_runner.tie_ok), on constructed logits."""
import numpy as np

from oracle_runner import DELTA_ROUTE, tie_ok


def test_exact_top_k_is_accepted():
    lg = np.array([0.5, 3.0, 2.0, -1.0, 1.0])
    assert tie_ok(lg, [1, 2, 4], 3)


def test_rank_swap_needs_a_near_tie():
    lg = np.array([0.5, 3.0, 2.0, 2.0 + 0.5 * DELTA_ROUTE, 1.0])
    assert tie_ok(lg, [1, 2, 3], 3)          # 2 and 3 within the tolerance: either order
    assert tie_ok(lg, [1, 3, 2], 3)
    lg2 = np.array([0.5, 3.0, 2.0, 2.1, 1.0])
    assert not tie_ok(lg2, [1, 2, 3], 3)     # a clear inversion


def test_membership_swap_needs_a_near_tie():
    lg = np.array([0.5, 3.0, 2.0, 1.0, 1.0 - 0.5 * DELTA_ROUTE])
    assert tie_ok(lg, [1, 2, 4], 3)          # the k-th and (k+1)-th are within the tolerance
    assert not tie_ok(lg, [1, 2, 0], 3)      # expert 0 is far below the k-th logit


def test_duplicates_and_wrong_count_are_rejected():
    lg = np.array([3.0, 2.0, 1.0])
    assert not tie_ok(lg, [0, 0], 2)
    assert not tie_ok(lg, [0], 2)
