"""CPU checks of the C ABI: the library loads, exports every function the headers
declare, and the host tree builder equals the oracle's tree buffers (no GPU needed)."""
import ctypes as C
import glob
import os
import re

import numpy as np
import pytest

from oracle.tree import anc_bits, tree_buffers
from workloads import PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, chain_choices, choices_to_arrays, seeded_tree_choices

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from speculative_decoding_heads_amd import _lib as L
    return L, L.lib()


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        for m in re.finditer(r"\b([A-Za-z_]\w*)\s*\(([^;{}()]*)\)\s*;", src):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported():
    L, lib = _lib()
    declared = _declared_functions()
    assert len(declared) >= 25
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert set(L.EXPORTED) >= {"medusa_heads_topk", "tree_build_candidates", "tree_attention",
                               "evaluate_posterior", "kv_compact"}
    assert set(L.EXPORTED) <= declared


def _host_tree(choices, K=0):
    L, lib = _lib()
    r, o = choices_to_arrays(choices)
    if len(r) == 0:
        r = np.zeros(1, np.int32)
    h = L.TreeHost()
    rc = lib.medusa_tree_build_host(r.ctypes.data, o.ctypes.data, len(choices), K, C.byref(h))
    return rc, h


@pytest.mark.parametrize("choices", [PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, seeded_tree_choices(0),
                                     seeded_tree_choices(4), chain_choices(1), chain_choices(63), []])
def test_host_tree_builder_matches_oracle(choices):
    rc, h = _host_tree(choices)
    assert rc == 0
    t = tree_buffers(choices) if choices else None
    if t is None:
        assert (h.T, h.P, h.D) == (1, 1, 0)
        assert h.anc[0] == 1 and h.retrieve[0] == 0
        return
    T, P, D = t["T"], t["P"], t["D"]
    assert (h.T, h.P, h.D, h.K) == (T, P, D, t["K"])
    assert list(h.tree_indices[:T]) == t["tree_indices"].tolist()
    assert list(h.depth[:T]) == t["depth"].tolist()
    assert list(h.parent[:T]) == t["parent"].tolist()
    assert [int(x) for x in h.anc[:T]] == [int(x) for x in anc_bits(t["anc"])]
    rt = np.array(h.retrieve).reshape(64, 64)[:P, : D + 1]
    assert rt.tolist() == t["retrieve"].tolist()
    assert list(h.path_len[:P]) == t["path_len"].tolist()


@pytest.mark.parametrize("bad,code", [([(0,), (0,)], -1), ([(0, 1)], -1), ([(-1,)], -1),
                                      ([(k,) for k in range(64)], -2)])
def test_host_tree_builder_rejects(bad, code):
    rc, _ = _host_tree(bad)
    assert rc == code


def test_rank_beyond_K_rejected():
    rc, _ = _host_tree([(0,), (3,)], K=3)
    assert rc == -1


def test_status_message_is_set():
    L, lib = _lib()
    _host_tree([(0,), (0,)])
    assert b"duplicate" in lib.medusa_last_error()
