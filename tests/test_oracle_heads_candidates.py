"""Pins of the oracle's Medusa heads, top-K and candidate expansion (CPU)."""
import json
import os

import numpy as np
import torch

from oracle.candidates import build_candidates
from oracle.heads import medusa_heads_logits, medusa_heads_topk, medusa_head_z, topk_desc
from oracle.tree import tree_buffers
from workloads import TWO_HEAD_CHOICES

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "heads_hand_example.json")))


def test_heads_hand_example():
    h, W1, W2 = (np.array(GOLD[k]) for k in ("h", "W1", "W2"))
    np.testing.assert_allclose(medusa_head_z(h, W1), GOLD["z"], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(medusa_heads_logits(h, W1, W2), GOLD["logits"], rtol=1e-15, atol=1e-15)
    idx, _ = medusa_heads_topk(h, W1, W2, 2)
    assert idx.tolist() == GOLD["top2"]


def test_zero_w1_reduces_to_projection_of_h():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((3, 16))
    W2 = rng.standard_normal((2, 40, 16))
    lg = medusa_heads_logits(h, np.zeros((2, 16, 16)), W2)
    for k in range(2):
        np.testing.assert_allclose(lg[:, k], h @ W2[k].T, rtol=1e-13)


def test_topk_matches_torch_on_distinct_values_and_ties_go_low():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 300))
    ref = torch.topk(torch.from_numpy(x), 10, dim=-1).indices.numpy()
    assert np.array_equal(topk_desc(x, 10), ref)
    tied = np.array([[1.0, 3.0, 3.0, 0.5, 3.0, 2.0]])
    assert topk_desc(tied, 4).tolist() == [[1, 2, 4, 5]]


def test_candidates_two_head_by_hand():
    t = tree_buffers(TWO_HEAD_CHOICES)
    assert t["K"] == 3
    tok, pos, cart = build_candidates(t, np.array([7]), np.array([[[10, 11, 12], [20, 21, 22]]]), np.array([40]))
    assert tok.tolist() == [[7, 10, 11, 20, 21, 22, 20, 21, 22]]
    assert pos.tolist() == [[40, 41, 41, 42, 42, 42, 42, 42, 42]]
    assert cart.tolist() == [[[7, 11, 22], [7, 11, 21], [7, 11, 20], [7, 10, 22], [7, 10, 21], [7, 10, 20]]]


def test_candidates_pad_with_zero():
    t = tree_buffers([(0,), (1,), (0, 0)])
    topk = np.array([[[8, 9], [30, 31]], [[3, 4], [40, 41]]])
    tok, pos, cart = build_candidates(t, np.array([5, 6]), topk, np.array([1, 2]))
    assert tok.tolist() == [[5, 8, 9, 30], [6, 3, 4, 40]]
    # paths: leaf 3 -> [0, 1, 3]; leaf 2 -> [0, 2, -1] (the pad picks token 0)
    assert cart.tolist() == [[[5, 8, 30], [5, 9, 0]], [[6, 3, 40], [6, 4, 0]]]
