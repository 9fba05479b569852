"""Pins of the kept-set acceptance rule (keptsets.py) on hand-made score
vectors: exact ties, a relative zone of 1e-6 around the k-th score, and the
+inf window. CPU only."""
import numpy as np

from keptsets import check_kept


def test_plateau_at_kth_score_any_member_accepted():
    S = np.array([5.0, 4.0, 3.0, 3.0, 3.0, 1.0])
    # oracle (ties to the newer token): {0, 1, 4}
    c = check_kept([0, 1, 4], S, 3)
    assert c.ok and c.same and c.n_zone == 3
    for alt in ([0, 1, 2], [1, 3, 0]):
        c = check_kept(alt, S, 3)
        assert c.ok and not c.same and c.n_diff == 2 and c.max_rel == 0.0


def test_above_zone_token_missing_or_below_zone_taken_is_rejected():
    S = np.array([5.0, 4.0, 3.0, 3.0, 3.0, 1.0])
    c = check_kept([0, 2, 3], S, 3)
    assert not c.ok and c.n_above_missing == 1
    c = check_kept([0, 1, 5], S, 3)
    assert not c.ok and c.n_below_taken == 1


def test_relative_zone_is_one_millionth_of_the_kth_score():
    # s_k = 1 + 5e-7 (2nd largest); zone half-width ~1.0000005e-6
    S = np.array([1.0, 1.0 + 5e-7, 1.0 + 2e-6, 0.5])
    assert check_kept([1, 2], S, 2).same
    c = check_kept([0, 2], S, 2)           # 1.0 lies 5e-7 below s_k: inside
    assert c.ok and not c.same and abs(c.max_rel - 5e-7 / (1 + 5e-7)) < 1e-12
    c = check_kept([0, 1], S, 2)           # 1 + 2e-6 lies above the zone: must be kept
    assert not c.ok and c.n_above_missing == 1
    # scaled scores: the zone scales with |s_k|
    assert check_kept([0, 2], S * 1e-3, 2).ok
    assert not check_kept([0, 1], S * 1e-3, 2).ok


def test_wrong_count_duplicates_or_range_rejected():
    S = np.array([3.0, 2.0, 1.0, 0.0])
    assert not check_kept([0, 1, 2], S, 2).ok
    assert not check_kept([0, 0], S, 2).ok
    assert not check_kept([0, 4], S, 2).ok


def test_window_infinities_and_negative_scores():
    S = np.array([-1.0, -2.0, -2.0 - 1e-7, -3.0, np.inf, np.inf])
    # k = 3: the window plus the best finite one
    assert check_kept([0, 4, 5], S, 3).same
    assert not check_kept([1, 4, 5], S, 3).ok
    # k = 4: s_k = -2, zone |S + 2| <= 2e-6 holds tokens 1 and 2
    assert check_kept([0, 2, 4, 5], S, 4).ok
    # k = 2: s_k = +inf, only the window
    assert check_kept([4, 5], S, 2).same
    assert not check_kept([0, 5], S, 2).ok
