"""Pins of the oracle's tree attention (CPU): special cases that reduce to textbook
causal attention / single-token decode computed by torch's scaled_dot_product_attention
in float64, the per-path equivalence of the tree mask, GQA head sharing, and convexity."""
import numpy as np
import pytest
import torch

from oracle.attention import attention_slice, tree_attention
from oracle.tree import chain_choices, tree_buffers
from workloads import PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, seeded_tree_choices


def _sdpa(q, k, v, mask, scale):
    """torch SDPA in float64: q [H, N, Dh], k/v [H, M, Dh], mask [N, M] bool (True = visible)."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy()


def _inputs(rng, B, T, Hq, Hkv, Dh, L):
    q = rng.standard_normal((B, T, Hq, Dh))
    Kc = rng.standard_normal((B, Hkv, L + 3, Dh))
    Vc = rng.standard_normal((B, Hkv, L + 3, Dh))
    Kt = rng.standard_normal((B, Hkv, T, Dh))
    Vt = rng.standard_normal((B, Hkv, T, Dh))
    return q, Kc, Vc, Kt, Vt


@pytest.mark.parametrize("L,n", [(0, 5), (7, 1), (33, 9), (100, 4)])
def test_chain_tree_equals_causal_attention(L, n):
    rng = np.random.default_rng(L * 10 + n)
    t = tree_buffers(chain_choices(n - 1)) if n > 1 else dict(anc=np.ones((1, 1), bool))
    T = n
    B, Hq, Hkv, Dh = 2, 4, 2, 8
    q, Kc, Vc, Kt, Vt = _inputs(rng, B, T, Hq, Hkv, Dh, L)
    seq = np.array([L, L])
    scale = 0.3
    out = tree_attention(q, Kc, Vc, seq, Kt, Vt, t["anc"], scale)
    # textbook causal attention over the concatenated sequence [prefix; chain]
    for b in range(B):
        k = np.concatenate([Kc[b, :, :L], Kt[b]], axis=1)  # [Hkv, L+T, Dh]
        v = np.concatenate([Vc[b, :, :L], Vt[b]], axis=1)
        k = np.repeat(k, Hq // Hkv, axis=0)
        v = np.repeat(v, Hq // Hkv, axis=0)
        causal = np.tril(np.ones((L + T, L + T), bool))[L:]  # rows of the last T positions
        ref = _sdpa(q[b].transpose(1, 0, 2).copy(), k, v, causal, scale)
        np.testing.assert_allclose(out[b].transpose(1, 0, 2), ref, rtol=1e-12, atol=1e-12)


def test_single_token_equals_decode():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, Dh, L = 3, 8, 8, 16, 50
    q, Kc, Vc, Kt, Vt = _inputs(rng, B, 1, Hq, Hkv, Dh, L)
    seq = np.array([50, 17, 1])
    out = tree_attention(q, Kc, Vc, seq, Kt, Vt, np.ones((1, 1), bool), 0.25)
    for b in range(B):
        Lb = seq[b]
        k = np.concatenate([Kc[b, :, :Lb], Kt[b]], axis=1)
        v = np.concatenate([Vc[b, :, :Lb], Vt[b]], axis=1)
        ref = _sdpa(q[b].transpose(1, 0, 2).copy(), k, v, np.ones((1, Lb + 1), bool), 0.25)
        np.testing.assert_allclose(out[b, 0], ref[:, 0], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("choices", [TWO_HEAD_CHOICES, PAGE_TREE_CHOICES, seeded_tree_choices(1)])
def test_tree_equals_causal_along_each_path(choices):
    """Tree attention of a node equals causal attention over prefix + its own root-to-node path."""
    t = tree_buffers(choices)
    rng = np.random.default_rng(11)
    T, Hq, Hkv, Dh, L = t["T"], 4, 1, 8, 20
    q, Kc, Vc, Kt, Vt = _inputs(rng, 1, T, Hq, Hkv, Dh, L)
    out = tree_attention(q, Kc, Vc, np.array([L]), Kt, Vt, t["anc"], 0.35)
    for p in range(t["P"]):
        nodes = t["retrieve"][p, : t["path_len"][p]]
        k = np.concatenate([Kc[0, :, :L], Kt[0][:, nodes]], axis=1)
        v = np.concatenate([Vc[0, :, :L], Vt[0][:, nodes]], axis=1)
        k, v = np.repeat(k, Hq, 0), np.repeat(v, Hq, 0)
        n = len(nodes)
        causal = np.tril(np.ones((L + n, L + n), bool))[L:]
        ref = _sdpa(q[0][nodes].transpose(1, 0, 2).copy(), k, v, causal, 0.35)
        np.testing.assert_allclose(out[0][nodes].transpose(1, 0, 2), ref, rtol=1e-12, atol=1e-12)


def test_gqa_sharing_and_convexity():
    rng = np.random.default_rng(2)
    t = tree_buffers(TWO_HEAD_CHOICES)
    q, Kc, Vc, Kt, Vt = _inputs(rng, 1, 9, 6, 2, 4, 12)
    seq = np.array([12])
    out = tree_attention(q, Kc, Vc, seq, Kt, Vt, t["anc"], 0.5)
    # query head h uses KV head h // 3
    for h in range(6):
        g = h // 3
        ref = attention_slice(q[0][:, h:h + 1], Kc[0, g, :12], Vc[0, g, :12], Kt[0, g], Vt[0, g], t["anc"], 0.5)
        np.testing.assert_allclose(out[0][:, h:h + 1], ref, rtol=0, atol=0)
    # constant values -> output is that constant (weights sum to one)
    ones = tree_attention(q, Kc, np.ones_like(Vc) * 2.5, seq, Kt, np.ones_like(Vt) * 2.5, t["anc"], 0.5)
    np.testing.assert_allclose(ones, 2.5, rtol=1e-14)


def test_cache_tail_is_ignored():
    rng = np.random.default_rng(3)
    t = tree_buffers(TWO_HEAD_CHOICES)
    q, Kc, Vc, Kt, Vt = _inputs(rng, 1, 9, 2, 2, 4, 10)
    Kc[:, :, 10:] = np.nan
    Vc[:, :, 10:] = np.nan
    out = tree_attention(q, Kc, Vc, np.array([10]), Kt, Vt, t["anc"], 0.5)
    assert np.isfinite(out).all()
