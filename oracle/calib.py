"""Tree calibration: the static sparse tree from per-(depth, rank) acceptance rates.

Follows "大模型推理 memory bandwidth bound (5) - Medusa", section 一.2: the
candidate tree is sparse and built ahead of time, keeping the candidate paths
of high probability and dropping the many of low probability, and the figure
there shows the accepted length growing with the candidate count while the
speed peaks and then falls.  The page gives no construction, so this module
takes the plainest reading that fits it:

* the true token at depth d (the token head d predicts) sits at rank r of that
  head's top-K with probability ``acc[d][r]``, the ranks of one depth being
  mutually exclusive (``sum_r acc[d][r] <= 1``) and the depths independent;
* a node's path probability is the product of ``acc`` along its rank path, and
  the expected number of accepted candidate tokens of a tree is the sum of its
  nodes' path probabilities (the accepted prefix of the true rank sequence has
  length l exactly when its first l ranks form a tree path, so the expected
  length is the sum over l of P(the first l true ranks are a path of the tree));
* the tree of n nodes (root included) with the largest expected length is the
  root plus the n - 1 most probable paths: a path is never more probable than
  its parent path, so the most probable paths are prefix-closed.  Ties go to
  the shorter path, then to the lexicographically smaller ranks, so a parent
  always precedes its children of equal probability.

``head_hit_counts`` is the teacher-forced measurement that produces such a
table: at every position t of a token sequence, head k's top-K (taken at the
hidden state of token t) is compared with the token k + 1 places further on
(the LM head predicts the next token, head 1 the one after it).

Test infrastructure only (see ``oracle/__init__``).
"""
import itertools

import numpy as np


def path_probability(path, acc):
    """Product of acc[depth][rank] along a rank path, multiplied from depth 0 up."""
    p = 1.0
    for d, r in enumerate(path):
        p = p * float(acc[d][r])
    return p


def expected_accept_length(choices, acc):
    """Expected accepted candidate tokens of a tree (the root's token not counted)."""
    return sum(path_probability(c, acc) for c in choices)


def best_tree(acc, n_nodes):
    """The n_nodes - 1 most probable rank paths (ties: shorter, then smaller ranks).

    acc: [H][K] table; paths up to depth H, ranks below K.  Every path of the
    full K-ary tree of depth H is scored and the best n_nodes - 1 kept."""
    H, K = len(acc), len(acc[0])
    paths = []
    for depth in range(1, H + 1):
        for path in itertools.product(range(K), repeat=depth):
            paths.append(path)
    if n_nodes - 1 > len(paths):
        raise ValueError("more nodes than the full tree has")
    paths.sort(key=lambda c: (-path_probability(c, acc), len(c), c))
    return paths[: n_nodes - 1]


def head_hit_counts(topk, tokens):
    """Teacher-forced hits: counts[k][r] = #{t : topk[t][k][r] == tokens[t + k + 2]}.

    topk: [N, H, K] top-K of each head at the hidden state of tokens[t]
    tokens: [N + H + 1] token sequence (tokens[t + 1] is the LM head's target)
    Returns (counts [H, K] int64, positions [H] int64: the t with a target)."""
    topk = np.asarray(topk)
    tokens = np.asarray(tokens)
    N, H, K = topk.shape
    counts = np.zeros((H, K), np.int64)
    positions = np.zeros(H, np.int64)
    for t in range(N):
        for k in range(H):
            j = t + k + 2
            if j >= len(tokens):
                continue
            positions[k] += 1
            for r in range(K):
                if int(topk[t, k, r]) == int(tokens[j]):
                    counts[k, r] += 1
    return counts, positions
