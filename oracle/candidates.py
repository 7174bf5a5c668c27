"""Candidate expansion through the static tree.

Follows "大模型推理 memory bandwidth bound (5) - Medusa", section 二.4
``generate_candidates()``: the flat candidate list is the root token followed by
each head's top-K indices, ``tree_candidates = candidates[tree_indices]``, and
the cartesian paths gather the tree tokens by ``retrieve_indices`` after a 0 is
appended so that the -1 padding picks that 0.  Section 二.5 ``tree_decoding()``
gives the positions: ``depth + current sequence length``.

Test infrastructure only (see ``oracle/__init__``).
"""
import numpy as np


def flat_candidates(root, topk_idx):
    """[B, 1 + H*K]: root token, then head 1's top-K, ..., head H's top-K."""
    root = np.asarray(root, dtype=np.int64).reshape(-1, 1)
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    B = topk_idx.shape[0]
    return np.concatenate([root, topk_idx.reshape(B, -1)], axis=1)


def build_candidates(tree, root, topk_idx, seq_len):
    """(tree_tokens [B, T], tree_pos [B, T], cart [B, P, D+1]) for a batch."""
    flat = flat_candidates(root, topk_idx)
    B = flat.shape[0]
    tree_tokens = flat[:, tree["tree_indices"]]
    tree_pos = np.asarray(seq_len, dtype=np.int64).reshape(B, 1) + tree["depth"][None, :]
    ext = np.concatenate([tree_tokens, np.zeros((B, 1), dtype=np.int64)], axis=1)
    cart = ext[:, tree["retrieve"]]  # index -1 selects the appended 0
    return tree_tokens, tree_pos, cart
