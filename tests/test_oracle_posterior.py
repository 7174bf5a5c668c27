"""Pins of the oracle's acceptance rule (CPU): hand-built greedy cases, closed-form
typical thresholds on uniform / two-point distributions, the eps/temperature
special cases, the padding reading, and a cross-check against a node-by-node
reachability formulation of the same rule."""
import math

import numpy as np
import pytest

from oracle.posterior import GREEDY, TYPICAL, evaluate_posterior, evaluate_posterior_one
from oracle.tree import tree_buffers
from workloads import PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, seeded_tree_choices

TWO = tree_buffers(TWO_HEAD_CHOICES)  # retrieve rows: [0,2,8],[0,2,7],[0,2,6],[0,1,5],[0,1,4],[0,1,3]


def _onehot_logits(T, V, amax):
    lg = np.zeros((T, V))
    for u, a in enumerate(amax):
        lg[u, a] = 5.0
    return lg


def test_greedy_by_hand():
    toks = np.array([0, 10, 11, 20, 21, 22, 30, 31, 32])
    # argmax at root = token of node 2 (11); at node 2 = token of node 7 (31); node 7 -> 9
    amax = [11, 0, 31, 0, 0, 0, 0, 9, 0]
    r = evaluate_posterior_one(TWO, _onehot_logits(9, 40, amax), toks, GREEDY)
    assert (r["best"], r["accept_len"], r["sel"], r["next_root"]) == (1, 2, 7, 9)
    assert r["acc"].tolist() == [1, 2, 1, 0, 0, 0]


def test_greedy_first_path_on_equal_length():
    toks = np.array([0, 10, 11, 20, 21, 22, 30, 31, 31])  # nodes 7 and 8 carry the same token
    amax = [11, 0, 31, 0, 0, 0, 0, 3, 4]
    r = evaluate_posterior_one(TWO, _onehot_logits(9, 40, amax), toks, GREEDY)
    assert (r["best"], r["accept_len"], r["sel"], r["next_root"]) == (0, 2, 8, 4)


def test_greedy_nothing_accepted():
    toks = np.array([0, 10, 11, 20, 21, 22, 30, 31, 32])
    amax = [39, 0, 0, 0, 0, 0, 0, 0, 0]
    r = evaluate_posterior_one(TWO, _onehot_logits(9, 40, amax), toks, GREEDY)
    assert (r["best"], r["accept_len"], r["sel"], r["next_root"]) == (0, 0, 0, 39)


def test_padded_slot_is_never_accepted():
    t = tree_buffers([(0,), (1,), (0, 0)])  # paths [0,1,3], [0,2,-1]
    toks = np.array([3, 7, 8, 9])
    amax = [8, 1, 0, 1]  # node 2's argmax is token 0, the pad value
    r = evaluate_posterior_one(t, _onehot_logits(4, 12, amax), toks, GREEDY)
    assert (r["best"], r["accept_len"], r["sel"], r["next_root"]) == (1, 1, 2, 0)


def _uniform_case(V, eps, delta):
    lg = np.zeros((9, V))
    toks = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8]) % V
    return evaluate_posterior_one(TWO, lg, toks, TYPICAL, 0.7, eps, delta)


@pytest.mark.parametrize("V,eps,delta,accept", [
    (512, 0.09, 0.3, True),     # thr = 0.3 (1/512 + 1e-5) < 1/512
    (32000, 1.0, 0.9, False),   # the +1e-5 inside the log decides: 0.9 * 4.125e-5 > 3.125e-5
    (512, 0.003, 0.3, True),    # the smaller of the two bounds is used, not the larger
    (512, 0.001, 1.0, True),    # eps caps the threshold below 1/512 < 1/512 + 1e-5
    (512, 0.09, 1.0, False),    # 1/512 + 1e-5 > 1/512
])
def test_typical_uniform_closed_form(V, eps, delta, accept):
    # uniform q = 1/V: H' = -log(1/V + 1e-5) exactly, so exp(-H') = 1/V + 1e-5
    thr = min(eps, delta * (1.0 / V + 1e-5))
    assert (1.0 / V > thr) == accept
    r = _uniform_case(V, eps, delta)
    if accept:
        # every path accepted to full depth; equal likelihoods -> first path
        assert (r["best"], r["accept_len"], r["sel"], r["next_root"]) == (0, 2, 8, 0)
    else:
        assert (r["best"], r["accept_len"], r["sel"], r["next_root"]) == (0, 0, 0, 0)


def test_typical_temperature_is_applied():
    # logits [tau*ln3, 0] at tau = 0.5 give q = [3/4, 1/4]; with eps 0.3, delta 1 the
    # candidate token 1 (q = 1/4) is rejected; ignoring tau would give q = 0.366 > 0.3.
    tau = 0.5
    lg = np.zeros((9, 2))
    lg[:, 0] = tau * math.log(3.0)
    toks = np.ones(9, dtype=np.int64)
    r = evaluate_posterior_one(TWO, lg, toks, TYPICAL, tau, 0.3, 1.0)
    assert r["accept_len"] == 0
    toks0 = np.zeros(9, dtype=np.int64)  # token 0 (q = 3/4) is accepted everywhere
    r = evaluate_posterior_one(TWO, lg, toks0, TYPICAL, tau, 0.3, 1.0)
    assert r["accept_len"] == 2 and r["best"] == 0


def test_typical_likelihood_tiebreak_by_hand():
    # Root's distribution favours token 2 (node 2) over token 1 (node 1); below them every
    # candidate is accepted, so both depth-2 families tie on length and the likelihood decides.
    V = 8
    lg = np.zeros((9, V))
    lg[0, 1], lg[0, 2] = 2.0, 3.0
    toks = np.array([0, 1, 2, 3, 4, 5, 3, 4, 5])
    r = evaluate_posterior_one(TWO, lg, toks, TYPICAL, 1.0, 0.0, 0.3)  # eps 0 -> threshold 0
    assert r["accept_len"] == 2
    assert r["best"] == 0 and r["sel"] == 8  # first path under node 2


def test_eps_zero_accepts_everything_and_eps_one_nothing():
    rng = np.random.default_rng(4)
    t = tree_buffers(PAGE_TREE_CHOICES)
    lg = rng.standard_normal((64, 100))
    toks = rng.integers(0, 100, 64)
    r = evaluate_posterior_one(t, lg, toks, TYPICAL, 0.7, 0.0, 0.3)
    assert r["accept_len"] == t["D"]
    assert t["path_len"][r["best"]] == t["D"] + 1
    r = evaluate_posterior_one(t, lg, toks, TYPICAL, 0.7, 2.0, 1e6)
    assert (r["accept_len"], r["best"], r["sel"]) == (0, 0, 0)


def test_small_temperature_equals_greedy():
    rng = np.random.default_rng(8)
    t = tree_buffers(seeded_tree_choices(2))
    for trial in range(20):
        lg = rng.standard_normal((64, 50)) * 3
        amax = lg.argmax(1)
        toks = rng.integers(0, 50, 64)
        # make some children match their parent's argmax
        for c in range(1, 64):
            if rng.uniform() < 0.6:
                toks[c] = amax[t["parent"][c]]
        g = evaluate_posterior_one(t, lg, toks, GREEDY)
        ty = evaluate_posterior_one(t, lg, toks, TYPICAL, 1e-3, 0.09, 0.3)
        assert ty["accept_len"] == g["accept_len"]
        assert ty["sel"] == g["sel"]  # greedy's accepted prefix is unique


def _reachability_form(tree, logits, toks, mode, tau=0.7, eps=0.09, delta=0.3):
    """The acceptance rule restated node by node (an independent formulation of
    section 二.6 / 一.3, not a per-path computation): a node is reached when its
    parent is reached and its own candidate passes the test taken at the parent;
    the accepted length is the depth of the deepest reached node; the chosen path
    is one whose entry at that depth is a deepest reached node -- the first such
    path for greedy, for typical the one whose node has the largest summed log q
    along its chain (first on equal sums).  q comes from a log-sum-exp log-softmax
    and the entropy from those log-probabilities."""
    T, parent, depth = tree["T"], tree["parent"], tree["depth"]
    lg = np.asarray(logits, np.float64)
    if mode == TYPICAL:
        z = lg / tau
        zmax = z.max(axis=1, keepdims=True)
        logq = z - (zmax + np.log(np.exp(z - zmax).sum(axis=1, keepdims=True)))
        q = np.exp(logq)
        ent = -(q * np.log(q + 1e-5)).sum(axis=1)
        thr = np.minimum(eps, delta * np.exp(-ent))
    reached = np.zeros(T, bool)
    reached[0] = True
    chain = np.zeros(T)
    for c in range(1, T):  # nodes are numbered depth by depth: parent[c] < c
        u = parent[c]
        if not reached[u]:
            continue
        if mode == GREEDY:
            ok = toks[c] == int(np.argmax(lg[u]))
        else:
            ok = np.float32(q[u, toks[c]]) > np.float32(thr[u])
        if ok:
            reached[c] = True
            chain[c] = chain[u] + (logq[u, toks[c]] if mode == TYPICAL else 0.0)
    a = int(depth[reached].max())
    ret, plen = tree["retrieve"], tree["path_len"]
    ends = [p for p in range(tree["P"]) if plen[p] > a and reached[ret[p, a]]]
    if a == 0:
        best = 0
    elif mode == GREEDY:
        best = ends[0]
    else:
        best = max(ends, key=lambda p: (chain[ret[p, a]], -p))
    sel = int(ret[best, a])
    return best, a, sel, int(np.argmax(lg[sel]))


@pytest.mark.parametrize("mode", [GREEDY, TYPICAL])
def test_cross_check_against_node_reachability_form(mode):
    rng = np.random.default_rng(21 + mode)
    for choices in (PAGE_TREE_CHOICES, seeded_tree_choices(0), TWO_HEAD_CHOICES):
        t = tree_buffers(choices)
        T = t["T"]
        for trial in range(15):
            V = 64
            lg = rng.standard_normal((T, V)) * (4.0 if mode == GREEDY else 1.5)
            toks = rng.integers(0, V, T)
            amax = lg.argmax(1)
            for c in range(1, T):
                if rng.uniform() < 0.7:
                    toks[c] = amax[t["parent"][c]]
            r = evaluate_posterior_one(t, lg, toks, mode, 0.7, 0.09, 0.3)
            ref = _reachability_form(t, lg, toks, mode)
            assert (r["best"], r["accept_len"], r["sel"], r["next_root"]) == ref


def test_flip_hook_inverts_one_decision():
    """Inverting the decision on one node changes the outcome exactly as the rule says:
    rejecting a reached node's candidate ends that chain there."""
    t = tree_buffers(TWO_HEAD_CHOICES)
    toks = np.array([0, 10, 11, 20, 21, 22, 30, 31, 32])
    amax = [11, 0, 31, 0, 0, 0, 0, 9, 0]
    lg = _onehot_logits(9, 40, amax)
    r = evaluate_posterior_one(t, lg, toks, GREEDY, flip={7})
    assert (r["best"], r["accept_len"], r["sel"], r["next_root"]) == (0, 1, 2, 31)
    r = evaluate_posterior_one(t, lg, toks, GREEDY, flip={1})  # node 1 (token 10) now accepted at the root
    assert r["acc"].tolist() == [1, 2, 1, 1, 1, 1] and r["best"] == 1


def test_batch_wrapper():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((3, 9, 20))
    toks = rng.integers(0, 20, (3, 9))
    best, a, sel, nr, res = evaluate_posterior(TWO, lg, toks, GREEDY)
    for b in range(3):
        r = evaluate_posterior_one(TWO, lg[b], toks[b], GREEDY)
        assert (best[b], a[b], sel[b], nr[b]) == (r["best"], r["accept_len"], r["sel"], r["next_root"])
