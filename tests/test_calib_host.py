"""The host tree builder (medusa_tree_from_acceptance) against the oracle: the
same paths in the same order and the same expected length, bit for bit (both
multiply the rates from depth 0 up and add the chosen paths in selection order).
Host-only C calls: no GPU is touched."""
import numpy as np
import pytest

from oracle.calib import best_tree, expected_accept_length


def _table(seed, H, K, ties=False):
    rng = np.random.default_rng(seed)
    if ties:
        a = rng.integers(1, 4, (H, K)).astype(np.float64) / 16.0  # few distinct values: many equal paths
    else:
        a = rng.random((H, K)) ** 3
        a = a / a.sum(1, keepdims=True) * rng.uniform(0.3, 0.95, (H, 1))
    return a


@pytest.mark.parametrize("seed,H,K,n", [(0, 4, 10, 64), (1, 4, 10, 26), (2, 5, 8, 48), (3, 1, 10, 11),
                                        (4, 3, 3, 40), (5, 4, 10, 1), (6, 2, 2, 7), (7, 4, 10, 2)])
def test_tree_from_acceptance_matches_oracle(seed, H, K, n):
    from speculative_decoding_heads_amd import api
    acc = _table(seed, H, K)
    got, exp = api.tree_from_acceptance(acc, n)
    want = best_tree(acc, n)
    assert got == want
    assert exp == expected_accept_length(want, acc)


@pytest.mark.parametrize("seed", [10, 11, 12])
def test_tree_from_acceptance_ties(seed):
    from speculative_decoding_heads_amd import api
    acc = _table(seed, 3, 4, ties=True)
    got, exp = api.tree_from_acceptance(acc, 50)
    assert got == best_tree(acc, 50)


def test_tree_from_acceptance_builds_a_valid_tree():
    """The builder's output goes straight into the library's host tree builder."""
    import ctypes as C
    from speculative_decoding_heads_amd import _lib as L
    from speculative_decoding_heads_amd import api
    from oracle.tree import tree_buffers, validate_choices
    acc = _table(20, 4, 10)
    choices, _ = api.tree_from_acceptance(acc, 64)
    validate_choices(choices, max_nodes=64)
    ranks = np.array([r for c in choices for r in c], np.int32)
    offsets = np.array([0] + list(np.cumsum([len(c) for c in choices])), np.int32)
    info = L.TreeHost()
    L.check(L.lib().medusa_tree_build_host(ranks.ctypes.data, offsets.ctypes.data, len(choices), 10, C.byref(info)))
    ref = tree_buffers(choices, K=10)
    assert info.T == ref["T"] == 64 and info.K == 10 and info.P == ref["P"]


@pytest.mark.parametrize("bad", ["neg", "sum", "size", "nodes"])
def test_tree_from_acceptance_rejects(bad):
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import MedusaError
    acc = _table(30, 3, 4)
    n = 10
    if bad == "neg":
        acc[1, 2] = -0.1
    elif bad == "sum":
        acc[0] = 0.5
    elif bad == "size":
        acc = _table(31, 1, 3)
        n = 5  # the full tree of depth 1, K 3 has 3 paths
    else:
        n = 65
    with pytest.raises(MedusaError):
        api.tree_from_acceptance(acc, n)
