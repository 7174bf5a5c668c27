"""Pins of the tree-calibration oracle (CPU).

* expected accepted length: against an exact enumeration of every outcome of
  the per-depth true ranks (each depth: one of the K ranks or none), taking the
  longest accepted prefix directly from the tree, and against a closed form for
  the chain tree;
* best tree: against an exhaustive search over every prefix-closed tree of the
  same size on small tables (no larger expected length exists), plus
  prefix-closure and the tie order on a table with equal entries;
* head hit counts: a hand-made sequence with known hits."""
import itertools

import numpy as np
import pytest

from oracle.calib import best_tree, expected_accept_length, head_hit_counts, path_probability
from oracle.tree import validate_choices


def _table(seed, H, K):
    rng = np.random.default_rng(seed)
    a = rng.random((H, K)) ** 2
    a = a / a.sum(1, keepdims=True) * rng.uniform(0.5, 0.95, (H, 1))
    return a


def _enumerated_length(choices, acc):
    """E[accepted] by brute force over all joint outcomes of the true ranks."""
    H, K = acc.shape
    tree = set(tuple(c) for c in choices)
    total = 0.0
    for outcome in itertools.product(range(K + 1), repeat=H):  # rank K = "no rank of the top-K"
        p = 1.0
        for d, r in enumerate(outcome):
            p *= acc[d, r] if r < K else 1.0 - acc[d].sum()
        n = 0
        while n < H and outcome[n] < K and tuple(outcome[: n + 1]) in tree:
            n += 1
        total += p * n
    return total


@pytest.mark.parametrize("seed,H,K", [(0, 2, 3), (1, 3, 3), (2, 3, 4), (3, 4, 2)])
def test_expected_length_matches_enumeration(seed, H, K):
    acc = _table(seed, H, K)
    rng = np.random.default_rng(seed + 10)
    full = [p for d in range(1, H + 1) for p in itertools.product(range(K), repeat=d)]
    for _ in range(5):
        # a random prefix-closed tree: random paths plus all their prefixes
        pick = [full[i] for i in rng.choice(len(full), size=min(6, len(full)), replace=False)]
        choices = sorted({p[:l] for p in pick for l in range(1, len(p) + 1)}, key=lambda c: (len(c), c))
        validate_choices(choices)
        assert abs(expected_accept_length(choices, acc) - _enumerated_length(choices, acc)) < 1e-12


def test_chain_tree_closed_form():
    # top-1 chain of depth 4: E = a1 + a1 a2 + a1 a2 a3 + a1 a2 a3 a4
    acc = np.array([[0.6, 0.2], [0.5, 0.1], [0.4, 0.3], [0.3, 0.3]])
    chain = [(0,), (0, 0), (0, 0, 0), (0, 0, 0, 0)]
    want = 0.6 + 0.6 * 0.5 + 0.6 * 0.5 * 0.4 + 0.6 * 0.5 * 0.4 * 0.3
    assert abs(expected_accept_length(chain, acc) - want) < 1e-15
    assert path_probability((1, 0, 1), acc) == pytest.approx(0.2 * 0.5 * 0.3, rel=1e-15)


def _all_trees(H, K, size):
    full = [p for d in range(1, H + 1) for p in itertools.product(range(K), repeat=d)]
    for sub in itertools.combinations(full, size):
        s = set(sub)
        if all(len(c) == 1 or c[:-1] in s for c in sub):
            yield sub


@pytest.mark.parametrize("seed,H,K,n_nodes", [(0, 2, 3, 4), (1, 2, 3, 6), (2, 3, 2, 5), (3, 3, 3, 5), (4, 2, 4, 7)])
def test_best_tree_is_optimal(seed, H, K, n_nodes):
    acc = _table(seed, H, K)
    got = best_tree(acc, n_nodes)
    validate_choices(got)
    assert len(got) == n_nodes - 1
    best = max(expected_accept_length(t, acc) for t in _all_trees(H, K, n_nodes - 1))
    assert expected_accept_length(got, acc) >= best - 1e-12


def test_best_tree_ties_and_growth():
    # equal entries everywhere: ties go to shorter paths, then smaller ranks
    acc = np.full((3, 3), 0.3)
    assert best_tree(acc, 5) == [(0,), (1,), (2,), (0, 0)]
    # every larger tree contains the smaller one (paths ranked once)
    acc = _table(9, 4, 5)
    prev = []
    for n in range(2, 40, 3):
        t = best_tree(acc, n)
        validate_choices(t)
        assert t[: len(prev)] == prev
        prev = t


def test_head_hit_counts_hand_example():
    # tokens 0..7; heads H = 2, K = 3; position t predicts tokens[t + 2] (head 1) and tokens[t + 3] (head 2)
    tokens = [10, 11, 12, 13, 14, 15, 16]
    topk = np.array([
        [[12, 99, 98], [97, 13, 96]],   # t = 0: head 1 rank 0 hits 12, head 2 rank 1 hits 13
        [[95, 94, 13], [14, 93, 92]],   # t = 1: head 1 rank 2 hits 13, head 2 rank 0 hits 14
        [[91, 90, 89], [88, 87, 15]],   # t = 2: head 1 misses 14, head 2 rank 2 hits 15
        [[15, 86, 85], [84, 83, 82]],   # t = 3: head 1 rank 0 hits 15, head 2 misses 16
        [[16, 81, 80], [16, 79, 78]],   # t = 4: head 1 rank 0 hits 16, head 2 has no target (t + 3 = 7)
    ])
    counts, positions = head_hit_counts(topk, tokens)
    np.testing.assert_array_equal(counts, [[3, 0, 1], [1, 1, 1]])
    np.testing.assert_array_equal(positions, [5, 4])
