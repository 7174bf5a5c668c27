"""State update after acceptance: token append and KV compaction.

Follows "大模型推理 memory bandwidth bound (5) - Medusa", section 二.7
``update_inference_inputs()``: the accepted tokens are the chosen path's first
a+1 entries (the root is always kept); the KV rows of those path nodes are
copied to the positions right after the previous sequence end; the sequence
length grows by a+1.

Reading: the tree's K/V live in a side buffer [.., T, Dh] rather than in the
cache slots after the prefix, so the copy is side buffer -> cache; the final
cache contents are the same as the page's in-place copy.

Test infrastructure only (see ``oracle/__init__``).
"""
import numpy as np


def kv_compact(tree, Kc, Vc, Kt, Vt, best, accept_len, seq_len):
    """Kc, Vc [NL, B, Hkv, Lmax, Dh]; Kt, Vt [NL, B, Hkv, T, Dh].

    Returns new (Kc, Vc, seq_len) -- inputs are not modified.
    """
    Kc = np.array(Kc, copy=True)
    Vc = np.array(Vc, copy=True)
    seq_len = np.array(seq_len, dtype=np.int64, copy=True)
    B = Kc.shape[1]
    for b in range(B):
        a = int(accept_len[b])
        rows = tree["retrieve"][int(best[b]), : a + 1]
        s = int(seq_len[b])
        if s + a + 1 > Kc.shape[3]:
            raise ValueError("cache overflow")
        Kc[:, b, :, s:s + a + 1, :] = np.asarray(Kt)[:, b][:, :, rows, :]
        Vc[:, b, :, s:s + a + 1, :] = np.asarray(Vt)[:, b][:, :, rows, :]
        seq_len[b] = s + a + 1
    return Kc, Vc, seq_len


def accepted_tokens(cart, best, accept_len):
    """List (per sequence) of the a+1 tokens appended this step."""
    return [list(np.asarray(cart[b, int(best[b]), : int(accept_len[b]) + 1], dtype=np.int64))
            for b in range(cart.shape[0])]
