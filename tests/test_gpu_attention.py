"""GPU parity of tree_attention against the oracle (element by element).

Tolerances: bf16 outputs within 2e-2 relative / 1e-2 absolute, fp32 within 1e-5.
Cache rows beyond each sequence's length hold NaN, so any read of them shows."""
import numpy as np
import pytest

from oracle.attention import attention_slice, tree_attention as oracle_attn
from oracle.tree import chain_choices, tree_buffers
from workloads import PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, attention_inputs, seeded_tree_choices

from _gpu import anc_tensor, assert_close, say, to_dev, to_np

pytestmark = pytest.mark.gpu

BF16_TOL = dict(rtol=2e-2, atol=1e-2)
F32_TOL = dict(rtol=1e-5, atol=1e-5)


def _run(dev, choices, B, Hq, Hkv, Dh, L, Lmax, dtype_name, seed, ragged=False, L_hint=None):
    import torch
    from speculative_decoding_heads_amd import api
    say("tree_attention", dtype_name, "B", B, "T", len(choices) + 1, "Hq", Hq, "Hkv", Hkv, "Dh", Dh, "L", L,
        "Lmax", Lmax, "seed", seed)
    tdt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    tree = api.Tree(choices)
    T = tree.T
    q, Kc, Vc, Kt, Vt, seq = attention_inputs(seed, B, T, Hq, Hkv, Dh, L, Lmax, bf16=dtype_name == "bf16",
                                              ragged=ragged)
    scale = 1.0 / np.sqrt(Dh)
    out = api.tree_attention(to_dev(q, tdt, dev), to_dev(Kc, tdt, dev), to_dev(Vc, tdt, dev),
                             torch.from_numpy(seq).to(dev), to_dev(Kt, tdt, dev), to_dev(Vt, tdt, dev), tree, scale,
                             L_hint=L_hint)
    torch.cuda.synchronize()
    ref = oracle_attn(q, Kc, Vc, seq, Kt, Vt, tree_buffers(choices)["anc"] if choices else np.ones((1, 1), bool),
                      scale)
    return to_np(out), ref


@pytest.mark.parametrize("choices,B,Hq,Hkv,L,Lmax,ragged", [
    (PAGE_TREE_CHOICES, 2, 8, 2, 300, 320, True),       # ragged, several tiles, partial last tile
    (seeded_tree_choices(0), 1, 32, 8, 1024, 1024, False),  # the 1k-prefix kernel shape
    (TWO_HEAD_CHOICES, 3, 4, 4, 200, 256, True),         # MHA, small tree
    (PAGE_TREE_CHOICES, 1, 64, 8, 130, 192, False),      # G = 8: 512 rows -> two 256-row chunks
    ([], 2, 32, 8, 777, 800, True),                      # T = 1 decode
    (PAGE_TREE_CHOICES, 2, 8, 8, 0, 64, False),          # no prefix at all
    (PAGE_TREE_CHOICES, 2, 8, 4, 700, 768, True),        # G = 2: 128 rows, half the waves without rows
    (TWO_HEAD_CHOICES, 2, 32, 2, 333, 384, True),        # G = 16: 144 rows -> a partial 32-row block
    (chain_choices(11), 1, 32, 2, 2000, 2048, False),    # G = 16: 192 rows, a chain tree
    (seeded_tree_choices(0), 1, 32, 32, 1024, 1088, False),  # MHA 64 rows (7B shape)
    (seeded_tree_choices(0), 2, 32, 8, 1024, 1024, True),  # split KV over ragged 1k prefixes
    (seeded_tree_choices(0), 1, 32, 8, 16384, 16384, False),  # 4 waves, two row chunks, 16 splits
    (seeded_tree_choices(0), 8, 32, 8, 2048, 2048, True),  # batch 8: 4 waves, 2 splits
])
def test_bf16_mfma_parity(dev, choices, B, Hq, Hkv, L, Lmax, ragged):
    got, ref = _run(dev, choices, B, Hq, Hkv, 128, L, Lmax, "bf16", seed=L + B, ragged=ragged)
    assert_close(got, ref, what="bf16 Dh128", **BF16_TOL)


def test_bf16_mfma_dh64(dev):
    got, ref = _run(dev, seeded_tree_choices(1), 2, 16, 4, 64, 500, 512, "bf16", seed=5, ragged=True)
    assert_close(got, ref, what="bf16 Dh64", **BF16_TOL)


def test_bf16_many_splits(dev):
    # small unit count at a long prefix: the split-KV path with many partials
    got, ref = _run(dev, PAGE_TREE_CHOICES, 1, 4, 1, 128, 8192, 8192, "bf16", seed=9)
    assert_close(got, ref, what="bf16 splits", **BF16_TOL)


@pytest.mark.parametrize("lens", [(8192, 300), (0, 5000)])
def test_bf16_splits_without_prefix_tiles(dev, lens):
    """The split plan follows L_hint (8192); a sequence much shorter than it leaves
    splits with no prefix tile at all (only the last split holds the tree tile), whose
    empty partials the merge must weigh zero.  Cache rows past each length are NaN."""
    import torch
    from speculative_decoding_heads_amd import api
    say("tree_attention empty splits", lens)
    B, Hq, Hkv, Dh, Lmax = 2, 32, 8, 128, 8192
    tree = api.Tree(seeded_tree_choices(0))
    q, Kc, Vc, Kt, Vt, _ = attention_inputs(31, B, tree.T, Hq, Hkv, Dh, Lmax, Lmax)
    seq = np.array(lens, np.int32)
    for b in range(B):
        Kc[b, :, seq[b]:] = np.nan
        Vc[b, :, seq[b]:] = np.nan
    assert api.tree_attention_workspace_size(1, B, tree.T, Hq, Hkv, Dh, Lmax) > 0  # a split plan
    scale = 1.0 / np.sqrt(Dh)
    out = api.tree_attention(to_dev(q, torch.bfloat16, dev), to_dev(Kc, torch.bfloat16, dev),
                             to_dev(Vc, torch.bfloat16, dev), torch.from_numpy(seq).to(dev),
                             to_dev(Kt, torch.bfloat16, dev), to_dev(Vt, torch.bfloat16, dev), tree, scale,
                             L_hint=Lmax)
    torch.cuda.synchronize()
    ref = oracle_attn(q, Kc, Vc, seq, Kt, Vt, tree_buffers(seeded_tree_choices(0))["anc"], scale)
    assert_close(to_np(out), ref, what="bf16 empty splits", **BF16_TOL)


def test_bf16_generic_head_size(dev):
    got, ref = _run(dev, TWO_HEAD_CHOICES, 2, 8, 2, 32, 90, 100, "bf16", seed=3, ragged=True)
    assert_close(got, ref, what="bf16 generic", **BF16_TOL)


@pytest.mark.parametrize("choices,Dh", [(TWO_HEAD_CHOICES, 16), (PAGE_TREE_CHOICES, 64), (chain_choices(20), 128)])
def test_fp32_generic_parity(dev, choices, Dh):
    got, ref = _run(dev, choices, 2, 4, 2, Dh, 70, 80, "fp32", seed=Dh, ragged=True)
    assert_close(got, ref, what="fp32", **F32_TOL)


def test_chain_tree_matches_causal_prefill_mask(dev):
    """A chain tree and an explicit lower-triangular mask give the same result."""
    import torch
    from speculative_decoding_heads_amd import api
    say("tree_attention chain vs causal mask")
    n = 12
    q, Kc, Vc, Kt, Vt, seq = attention_inputs(11, 1, n, 8, 2, 128, 100, 128, bf16=True)
    args = [to_dev(x, torch.bfloat16, dev) for x in (q, Kc, Vc)]
    s = torch.from_numpy(seq).to(dev)
    kt, vt = to_dev(Kt, torch.bfloat16, dev), to_dev(Vt, torch.bfloat16, dev)
    a = api.tree_attention(*args, s, kt, vt, api.Tree(chain_choices(n - 1)), 0.1)
    b = api.tree_attention(*args, s, kt, vt, anc_tensor(np.tril(np.ones((n, n), bool)), dev), 0.1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_long_prefix_all_slices(dev):
    """Batch 8, 32/8 heads, prefix 65536: the long-context launch, checked against the
    oracle on all 64 (sequence, KV head) slices, one slice at a time."""
    import torch
    from speculative_decoding_heads_amd import api
    from workloads import torch_normal
    say("tree_attention long prefix B8 L65536")
    B, Hq, Hkv, Dh, L = 8, 32, 8, 128, 65536
    tree = api.Tree(seeded_tree_choices(0))
    T = tree.T
    q = torch_normal((B, T, Hq, Dh), 1.0, 101, dev, torch.bfloat16)
    Kc = torch_normal((B, Hkv, L, Dh), 1.0, 102, dev, torch.bfloat16)
    Vc = torch_normal((B, Hkv, L, Dh), 1.0, 103, dev, torch.bfloat16)
    Kt = torch_normal((B, Hkv, T, Dh), 1.0, 104, dev, torch.bfloat16)
    Vt = torch_normal((B, Hkv, T, Dh), 1.0, 105, dev, torch.bfloat16)
    seq = torch.full((B,), L, dtype=torch.int32, device=dev)
    seq[3] = L - 1000  # one ragged sequence
    out = api.tree_attention(q, Kc, Vc, seq, Kt, Vt, tree, 1.0 / np.sqrt(Dh))
    torch.cuda.synchronize()
    anc = tree_buffers(seeded_tree_choices(0))["anc"]
    G = Hq // Hkv
    for b in range(B):
        Lb = int(seq[b])
        for g in range(Hkv):
            ref = attention_slice(to_np(q[b, :, g * G:(g + 1) * G]), to_np(Kc[b, g, :Lb]), to_np(Vc[b, g, :Lb]),
                                  to_np(Kt[b, g]), to_np(Vt[b, g]), anc, 1.0 / np.sqrt(Dh))
            assert_close(to_np(out[b, :, g * G:(g + 1) * G]), ref, what="long slice %d,%d" % (b, g), **BF16_TOL)
