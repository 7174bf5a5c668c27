"""Pins of the oracle's tree buffers against the page's worked example and against
independent derivations (parent-pointer walks, counting), CPU only."""
import json
import os

import numpy as np
import pytest

from oracle.tree import anc_bits, chain_choices, dense_choices, tree_buffers, validate_choices
from workloads import PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, seeded_tree_choices

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_tree_buffers.json")))


def test_fixture_choices_match_workload_copy():
    assert [tuple(c) for c in GOLD["choices"]] == PAGE_TREE_CHOICES


def test_page_tree_sorted_and_sizes():
    t = tree_buffers(PAGE_TREE_CHOICES)
    assert [list(c) for c in t["sorted"]] == GOLD["sorted_choices"]
    assert t["T"] == GOLD["n_nodes"] == 64
    assert t["P"] == GOLD["n_paths"] == 42
    assert t["K"] == GOLD["topk"] == 10
    assert t["D"] == 4


def test_page_tree_indices_depth_retrieve():
    t = tree_buffers(PAGE_TREE_CHOICES)
    assert t["tree_indices"].tolist() == GOLD["tree_indices"]
    assert t["depth"].tolist() == GOLD["depth"]
    assert t["retrieve"].tolist() == GOLD["retrieve"]


def test_page_red_path_index_31():
    t = tree_buffers(PAGE_TREE_CHOICES)
    node = 1 + t["sorted"].index(tuple(GOLD["red_path_last_token"]["choice"]))
    assert t["tree_indices"][node] == GOLD["red_path_last_token"]["tree_index"]


def test_page_mask_corners():
    t = tree_buffers(PAGE_TREE_CHOICES)
    m = t["anc"].astype(int)
    c = GOLD["mask_corners"]
    for r in range(3):
        assert m[r, :3].tolist() + m[r, -3:].tolist() == c["rows_first"][r]
        assert m[61 + r, :3].tolist() + m[61 + r, -3:].tolist() == c["rows_last"][r]


def _anc_by_parent_walk(parent):
    T = len(parent)
    a = np.zeros((T, T), dtype=bool)
    for i in range(T):
        j = i
        while j >= 0:
            a[i, j] = True
            j = parent[j]
    return a


@pytest.mark.parametrize("choices", [PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, seeded_tree_choices(0),
                                     seeded_tree_choices(3), chain_choices(7), dense_choices((3, 2, 2))])
def test_mask_equals_ancestor_relation(choices):
    t = tree_buffers(choices)
    assert np.array_equal(t["anc"], _anc_by_parent_walk(t["parent"]))
    # lower triangular, root column full, popcount = depth + 1
    assert not np.triu(t["anc"], 1).any()
    assert t["anc"][:, 0].all()
    assert (t["anc"].sum(1) == t["depth"] + 1).all()
    # every retrieve row is a parent chain ending in a leaf
    for p in range(t["P"]):
        row = t["retrieve"][p, : t["path_len"][p]]
        assert row[0] == 0
        for j in range(1, len(row)):
            assert t["parent"][row[j]] == row[j - 1]
        assert (t["retrieve"][p, t["path_len"][p]:] == -1).all()
    # leaves = nodes that are nobody's parent; each appears in exactly one row
    leaves = sorted(set(range(t["T"])) - set(t["parent"][1:].tolist()), reverse=True)
    assert [int(t["retrieve"][p, t["path_len"][p] - 1]) for p in range(t["P"])] == leaves


def test_two_head_figure_row():
    """Section 一.2 figure: head 1 top-2 x head 2 top-3 gives 6 paths; the query 'is'
    on the path ['I', 'is'] (flattened row 6) sees only column 2 ('I') and itself."""
    t = tree_buffers(TWO_HEAD_CHOICES)
    assert t["P"] == 6 and t["T"] == 9
    assert np.flatnonzero(t["anc"][6]).tolist() == [0, 2, 6]


def test_chain_mask_is_causal():
    t = tree_buffers(chain_choices(10))
    assert np.array_equal(t["anc"], np.tril(np.ones((11, 11), dtype=bool)))
    assert t["P"] == 1


def test_anc_bits_roundtrip():
    t = tree_buffers(PAGE_TREE_CHOICES)
    bits = anc_bits(t["anc"])
    for i in range(64):
        for j in range(64):
            assert bool((int(bits[i]) >> j) & 1) == t["anc"][i, j]


def test_seeded_tree_is_greedy_frontier():
    """Every node in the seeded tree scores at least as much as any absent child of a tree node."""
    rng = np.random.default_rng(0)
    acc = np.sort(rng.uniform(0.0, 1.0, (4, 10)), axis=1)[:, ::-1]
    ch = seeded_tree_choices(0)
    validate_choices(ch, max_nodes=64)
    score = lambda c: float(np.prod([acc[d, r] for d, r in enumerate(c)]))
    s = set(ch)
    worst_in = min(score(c) for c in ch)
    frontier = [p + (r,) for p in [()] + ch for r in range(10) if len(p) < 4 and p + (r,) not in s]
    assert max(score(c) for c in frontier) <= worst_in
    t = tree_buffers(ch)
    assert t["T"] == 64 and t["D"] <= 4


@pytest.mark.parametrize("bad", [[(0,), (0,)], [(0, 1)], [(0,), (0, 0, 1)], [(-1,)]])
def test_invalid_choices_rejected(bad):
    with pytest.raises(ValueError):
        tree_buffers(bad)
