"""Medusa heads, per-head top-K and the root token.

Follows "大模型推理 memory bandwidth bound (5) - Medusa", section 一.1 (the head
is one residual block: p_t^(k) = softmax(W2^(k) (SiLU(W1^(k) h_t) + h_t)), with
W1 of size d x d) and section 二.4 ``generate_candidates()`` (the root is the
argmax of the LM-head logits at the last position when temperature is 0 or
``fast``; each head contributes the indices of its top-K logits).

Readings: the page writes W2 as "d x V" but applies it to a d-vector, so W2 is
stored [V, d] and ``logits = W2 @ z``; the heads carry no bias; top-K is taken on
the raw logits (softmax is monotone, the page's code also takes topk of the
logits), in value-descending order with ties going to the lower token index.
With ``bf16=True`` the residual-block output z is rounded to bfloat16 before
the V-projection, the storage point of the product path.

Test infrastructure only (see ``oracle/__init__``).
"""
import numpy as np

from .numerics import argmax_first, round_bf16, silu


def medusa_head_z(h, W1):
    """z[b, k, :] = h[b] + SiLU(W1[k] @ h[b]) for h [B, d], W1 [H, d, d]."""
    h = np.asarray(h, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    u = np.einsum("kij,bj->bki", W1, h)
    return h[:, None, :] + silu(u)


def medusa_heads_logits(h, W1, W2, bf16=False):
    """Logits [B, H, V] of every Medusa head.  W2 is [H, V, d].

    One head's W2 is converted to float64 at a time so the full-size workload
    (4 heads x 32000 x 4096) fits in host memory.
    """
    z = medusa_head_z(h, W1)
    if bf16:
        z = round_bf16(z)
    B, H, d = z.shape
    V = W2.shape[1]
    out = np.empty((B, H, V), dtype=np.float64)
    for k in range(H):
        out[:, k, :] = z[:, k, :] @ np.asarray(W2[k], dtype=np.float64).T
    return out


def topk_desc(values, K):
    """Indices of the K largest entries along the last axis, value-descending,
    ties to the lower index (a full stable sort, not a partial selection)."""
    v = np.asarray(values)
    flat = v.reshape(-1, v.shape[-1])
    out = np.empty((flat.shape[0], K), dtype=np.int64)
    idx = np.arange(v.shape[-1])
    for r in range(flat.shape[0]):
        order = np.lexsort((idx, -flat[r]))  # primary: -value, secondary: index
        out[r] = order[:K]
    return out.reshape(v.shape[:-1] + (K,))


def medusa_heads_topk(h, W1, W2, K, bf16=False):
    """(topk_idx [B, H, K], logits [B, H, V]) of the Medusa heads."""
    logits = medusa_heads_logits(h, W1, W2, bf16=bf16)
    return topk_desc(logits, K), logits


def root_token(last_logits):
    """Greedy root token: argmax of the LM-head logits, lowest index on ties."""
    return argmax_first(last_logits, axis=-1)
