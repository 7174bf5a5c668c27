"""Tree configurations (``medusa_choices`` rank-path lists) used as inputs.

* ``PAGE_TREE_CHOICES``: the 63-choice, 64-node sparse tree printed on the page
  "大模型推理 memory bandwidth bound (5) - Medusa", section 二.2 (the input of
  ``generate_medusa_buffers()``), in the page's order.
* ``TWO_HEAD_CHOICES``: the dense tree of the 2-head figure in section 一.2 of
  the same page (head 1 top-2, head 2 top-3: 8 non-root nodes, 6 paths).
* ``seeded_tree_choices``: a synthetic 64-node tree of depth <= 4 drawn from a
  seed -- per-(depth, rank) acceptance probabilities decreasing in rank, and the
  nodes added greedily by the largest product of probabilities along the path.
* ``chain_choices``: one rank-0 node per depth (the tree whose mask is causal).
"""
import itertools

import numpy as np

__all__ = ["PAGE_TREE_CHOICES", "TWO_HEAD_CHOICES", "seeded_tree_choices", "chain_choices",
           "choices_to_arrays", "acceptance_table"]

PAGE_TREE_CHOICES = [
    (0,), (0, 0), (1,), (0, 1), (0, 0, 0), (1, 0), (2,), (0, 2), (0, 0, 1), (0, 3), (3,),
    (0, 1, 0), (2, 0), (4,), (0, 0, 2), (0, 4), (1, 1), (1, 0, 0), (0, 0, 0, 0), (5,),
    (0, 0, 3), (0, 5), (0, 2, 0), (3, 0), (0, 1, 1), (0, 6), (6,), (0, 7), (0, 0, 4), (4, 0),
    (1, 2), (0, 8), (7,), (0, 3, 0), (0, 0, 0, 1), (0, 0, 5), (2, 1), (0, 0, 6), (1, 0, 1),
    (0, 0, 1, 0), (2, 0, 0), (5, 0), (0, 9), (0, 1, 2), (8,), (0, 4, 0), (0, 2, 1), (1, 3),
    (0, 0, 7), (0, 0, 0, 2), (0, 0, 8), (1, 1, 0), (0, 1, 0, 0), (6, 0), (9,), (0, 1, 3),
    (0, 0, 0, 3), (1, 0, 2), (0, 5, 0), (3, 1), (0, 0, 2, 0), (7, 0), (1, 4),
]

TWO_HEAD_CHOICES = [(0,), (1,), (0, 0), (0, 1), (0, 2), (1, 0), (1, 1), (1, 2)]


def chain_choices(n):
    return [tuple([0] * k) for k in range(1, n + 1)]


def seeded_tree_choices(seed=0, depth=4, topk=10, n_nodes=63):
    """Synthetic sparse tree: n_nodes rank paths (root excluded).

    Per depth, ``topk`` acceptance probabilities are drawn U(0, 1) and sorted in
    decreasing order (rank 0 is the most likely).  A path's score is the product
    of its per-depth probabilities; since every factor is below 1 a path scores
    below its prefix, so taking the n_nodes best-scoring paths (ties broken by
    depth, then ranks) is the same as greedily adding the best child, and the
    result is prefix-closed.
    """
    rng = np.random.default_rng(seed)
    acc = np.sort(rng.uniform(0.0, 1.0, (depth, topk)), axis=1)[:, ::-1]
    paths = []
    for d in range(1, depth + 1):
        for ranks in itertools.product(range(topk), repeat=d):
            score = 1.0
            for lvl, r in enumerate(ranks):
                score *= acc[lvl, r]
            paths.append((-score, d, ranks))
    paths.sort()
    return [p[2] for p in paths[:n_nodes]]


def choices_to_arrays(choices):
    """Flatten a choice list into (ranks int32 [sum len], offsets int32 [n+1]) for the C ABI."""
    ranks, offsets = [], [0]
    for c in choices:
        ranks.extend(int(r) for r in c)
        offsets.append(len(ranks))
    return np.asarray(ranks, dtype=np.int32), np.asarray(offsets, dtype=np.int32)


def acceptance_table(H, K, top=0.75, depth_decay=0.85, rank_ratio=0.5):
    """Synthetic per-(depth, rank) acceptance rates [H, K] (the pages print none):
    depth d's true token is in the top-K with probability top * depth_decay**d,
    split over the ranks in proportion to rank_ratio**r."""
    w = rank_ratio ** np.arange(K, dtype=np.float64)
    cover = top * depth_decay ** np.arange(H, dtype=np.float64)
    return cover[:, None] * (w / w.sum())[None, :]
