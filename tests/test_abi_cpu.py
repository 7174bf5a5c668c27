"""CPU checks of the C ABI: the library loads, exports every function the headers
declare, the host tree builder equals the oracle's tree buffers, and the attention
launch plan picks the measured split counts (no GPU needed)."""
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


@pytest.mark.parametrize("B,Hq,Hkv,L,splits", [
    (1, 32, 8, 1024, 4),    # 2 waves x 4 row chunks, 4 splits: 128 workgroups, none fills the chip
    (1, 32, 8, 2048, 8),    # 2 waves, 8 splits of 4 tiles: 256 workgroups
    (1, 32, 8, 16384, 16),  # 4 waves (2 row chunks), 16 splits of 16 tiles
    (1, 32, 8, 65536, 32),  # 8 waves, 32 splits of 32 tiles
    (8, 32, 8, 1024, 1),    # batch 8: 2 waves x 4 row chunks fill the chip unsplit
    (8, 32, 8, 2048, 2),    # 4 waves, 2 splits of 16 tiles
    (8, 32, 8, 65536, 4),   # 8 waves, 4 splits
    (1, 32, 32, 1152, 4),   # 32 KV heads, 18 tiles: at least 4 tiles a split
    (1, 32, 32, 65536, 8),  # 32 KV heads, 8 splits fill the chip
])
def test_attention_launch_plan_splits(B, Hq, Hkv, L, splits):
    """The KV split count of the bf16 attention launch plan (a 64-node tree, head size
    128), read back from the workspace size: fp32 partials of every query row of every
    split plus their maxima and sums, none when unsplit."""
    _, lib = _lib()
    T, Dh = 64, 128
    R = T * (Hq // Hkv)

    def up(x):
        return (x + 255) // 256 * 256

    expect = 0 if splits == 1 else up(B * Hkv * splits * R * Dh * 4) + up(B * Hkv * splits * R * 2 * 4)
    assert lib.tree_attention_workspace_size(1, B, T, Hq, Hkv, Dh, L) == expect
