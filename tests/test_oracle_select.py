"""Pins of the Viterbi selector: brute force over every path, special cases (CPU)."""
import time

import numpy as np
import pytest

from oracle import select


def random_problem(seed, P, K, V, r, s):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(P)])
    lp = np.sort(rng.standard_normal((P, K)) - 5.0, axis=1)[:, ::-1]
    A = rng.standard_normal((V, r)) * 0.3
    B = rng.standard_normal((V, r)) * 0.3
    return ids, lp, select.pair_scores(ids, A, B, s)


@pytest.mark.parametrize("seed", range(6))
def test_viterbi_equals_brute_force_top4(seed):
    """K = 4 candidates over 7 positions: all 16,384 paths."""
    ids, lp, T = random_problem(seed, 7, 4, 4096, 32, 1 / np.sqrt(32))
    path, best = select.viterbi(lp, T)
    bp, bb, second = select.brute_force(lp, T)
    assert np.array_equal(path, bp)
    assert np.isclose(best, bb, rtol=0, atol=1e-12)
    assert np.isclose(select.path_score(lp, T, path), best, atol=1e-12)


@pytest.mark.slow
def test_viterbi_equals_brute_force_top16_all_paths():
    """K = 16 over 7 positions: all 16^7 = 268,435,456 paths on a tiny vocabulary."""
    t0 = time.time()
    ids, lp, T = random_problem(11, 7, 16, 64, 8, 1 / np.sqrt(8))
    path, best = select.viterbi(lp, T)
    bp, bb, second = select.brute_force(lp, T)
    assert np.array_equal(path, bp)
    assert np.isclose(best, bb, atol=1e-12)
    assert bb > second
    assert time.time() - t0 < 300


def test_zero_pair_scale_is_per_position_argmax():
    rng = np.random.default_rng(3)
    lp = rng.standard_normal((7, 16))
    path, _ = select.viterbi(lp, np.zeros((6, 16, 16)))
    assert np.array_equal(path, lp.argmax(1))


def test_per_position_shift_invariance():
    """Adding a constant per position (e.g. the log-sum-exp) never changes the path."""
    ids, lp, T = random_problem(4, 7, 16, 1000, 16, 0.25)
    path, _ = select.viterbi(lp, T)
    shift = np.random.default_rng(9).standard_normal(7)[:, None] * 100
    path2, _ = select.viterbi(lp + shift, T)
    assert np.array_equal(path, path2)


def test_tie_rule_lowest_index():
    """Exact ties (dyadic values): lowest final index, lowest predecessors."""
    lp = np.zeros((4, 3))
    T = np.zeros((3, 3, 3))
    path, best = select.viterbi(lp, T)
    assert list(path) == [0, 0, 0, 0] and best == 0
    bp, _, _ = select.brute_force(lp, T)
    assert list(bp) == [0, 0, 0, 0]
    lp2 = np.array([[0, 1, 1.0], [0, 0, 0], [0, 0, 0], [0, 0.5, 0.5]])
    path, _ = select.viterbi(lp2, T)
    bp, _, _ = select.brute_force(lp2, T)
    assert list(path) == [1, 0, 0, 1] == list(bp)


def test_transition_direction():
    """The pair score reads A for the earlier position and B for the later one."""
    V, r = 6, 2
    A = np.zeros((V, r))
    B = np.zeros((V, r))
    A[1] = [1, 0]
    B[4] = [1, 0]
    ids = np.array([[0, 1], [3, 4], [5, 2]])
    T = select.pair_scores(ids, A, B, 2.0)
    assert T[0, 1, 1] == 2.0 and T[0].sum() == 2.0
    assert np.all(T[1] == 0)
    # and swapping the roles changes the score
    T2 = select.pair_scores(ids, B, A, 2.0)
    assert T2[0].sum() == 0.0
