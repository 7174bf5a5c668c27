"""Tree attention: T tree queries over the KV prefix plus the tree's own KV.

Follows "大模型推理 memory bandwidth bound (5) - Medusa", section 一.2 (the tree
is flattened into one sequence and the attention mask lets each node see only
its predecessors on its own path) and section 二.2 (``medusa_attn_mask``, root
column all ones), together with section 二.3 (the mask is installed on the base
model, so every cached prefix token stays visible to every tree node).

For query node i and query head h (KV head h // (Hq/Hkv), grouped-query
sharing):  out = softmax(scale * q . k over {prefix keys 0..seq_len-1} u
{tree keys j : anc[i, j]}) @ v, computed exactly with two passes in float64.

Test infrastructure only (see ``oracle/__init__``).
"""
import numpy as np


def attention_slice(q, Kp, Vp, Kt, Vt, anc, scale):
    """One (sequence, KV head) slice.

    q  [T, G, Dh]   the G query heads sharing this KV head, per tree node
    Kp, Vp [L, Dh]  the valid prefix rows only
    Kt, Vt [T, Dh]  the tree's own keys/values
    anc [T, T] bool
    returns [T, G, Dh] float64
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.concatenate([np.asarray(Kp, np.float64), np.asarray(Kt, np.float64)], axis=0)
    V = np.concatenate([np.asarray(Vp, np.float64), np.asarray(Vt, np.float64)], axis=0)
    L = Kp.shape[0]
    T, G, Dh = q.shape
    visible = np.concatenate([np.ones((T, L), dtype=bool), np.asarray(anc, dtype=bool)], axis=1)
    # scores of every (node, head) row against every key: one matrix product
    s = (q.reshape(T * G, Dh) @ K.T).reshape(T, G, -1) * scale
    s = np.where(visible[:, None, :], s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    p /= np.sum(p, axis=-1, keepdims=True)
    return (p.reshape(T * G, -1) @ V).reshape(T, G, Dh)


def tree_attention(q, Kc, Vc, seq_len, Kt, Vt, anc, scale):
    """Whole batch.

    q  [B, T, Hq, Dh];  Kc, Vc [B, Hkv, Lmax, Dh] (rows >= seq_len[b] ignored);
    Kt, Vt [B, Hkv, T, Dh];  anc [T, T] bool  ->  out [B, T, Hq, Dh] float64
    """
    q = np.asarray(q)
    B, T, Hq, Dh = q.shape
    Hkv = Kc.shape[1]
    G = Hq // Hkv
    out = np.empty((B, T, Hq, Dh), dtype=np.float64)
    for b in range(B):
        L = int(seq_len[b])
        for g in range(Hkv):
            out[b, :, g * G:(g + 1) * G, :] = attention_slice(
                q[b, :, g * G:(g + 1) * G, :], Kc[b, g, :L], Vc[b, g, :L],
                Kt[b, g], Vt[b, g], anc, scale)
    return out
