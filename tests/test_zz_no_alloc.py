"""tree_attention_noalloc (the split partials in the library's fixed device scratch,
no workspace argument) against tree_attention with a caller workspace: identical
outputs, bit for bit, on two calls in a row -- the batch-8 / prefix-65536 launch
(33.5 MB of partials) and then a smaller ragged one that reuses the same scratch."""
import numpy as np
import pytest

from workloads import PAGE_TREE_CHOICES, seeded_tree_choices, torch_normal

from _gpu import say

pytestmark = pytest.mark.gpu


def _inputs(dev, B, Hq, Hkv, Dh, L, T, seed, ragged):
    import torch
    q = torch_normal((B, T, Hq, Dh), 1.0, seed, dev, torch.bfloat16)
    Kc = torch_normal((B, Hkv, L, Dh), 1.0, seed + 1, dev, torch.bfloat16)
    Vc = torch_normal((B, Hkv, L, Dh), 1.0, seed + 2, dev, torch.bfloat16)
    Kt = torch_normal((B, Hkv, T, Dh), 1.0, seed + 3, dev, torch.bfloat16)
    Vt = torch_normal((B, Hkv, T, Dh), 1.0, seed + 4, dev, torch.bfloat16)
    seq = torch.full((B,), L, dtype=torch.int32, device=dev)
    if ragged:
        seq[1:] = torch.tensor([L - 1 - 37 * i for i in range(1, B)], dtype=torch.int32)
    return q, Kc, Vc, Kt, Vt, seq


def test_noalloc_matches_workspace_path_twice(dev):
    import torch
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import lib
    cap = lib().tree_attention_noalloc_max_scratch()
    cases = [(8, 32, 8, 128, 65536, seeded_tree_choices(0), 201, False),   # 33.5 MB of split partials
             (2, 16, 4, 128, 3000, PAGE_TREE_CHOICES, 301, True)]          # smaller, ragged
    for B, Hq, Hkv, Dh, L, choices, seed, ragged in cases:
        say("tree_attention_noalloc B", B, "Hq", Hq, "Hkv", Hkv, "L", L)
        tree = api.Tree(choices)
        need = api.tree_attention_workspace_size(1, B, tree.T, Hq, Hkv, Dh, L)
        assert 0 < need <= cap
        q, Kc, Vc, Kt, Vt, seq = _inputs(dev, B, Hq, Hkv, Dh, L, tree.T, seed, ragged)
        scale = 1.0 / np.sqrt(Dh)
        ref = api.tree_attention(q, Kc, Vc, seq, Kt, Vt, tree, scale)
        got = api.tree_attention_noalloc(q, Kc, Vc, seq, Kt, Vt, tree, scale)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, ref), "no-alloc output differs from the workspace path (B %d, L %d)" % (B, L)
        del q, Kc, Vc, Kt, Vt
        torch.cuda.empty_cache()
