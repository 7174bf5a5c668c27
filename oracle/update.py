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


def appended_counts(cart, best, accept_len, stop_token, done, n_out, max_new, seq_len, Lmax):
    """Per-sequence stop (reading of the page's medusa_generate loop, section 二.1,
    which ends generation once the end-of-sequence token is among the new tokens):
    a sequence appends its a+1 accepted tokens up to and including the first
    stop token, and no more than its remaining output room (max_new - n_out) and
    cache room (Lmax - seq_len); a finished sequence appends nothing.  A sequence
    finishes when it appends the stop token or its count reaches its room.
    Returns (counts, done')."""
    B = cart.shape[0]
    counts = np.zeros(B, dtype=np.int64)
    new_done = np.array(done, dtype=bool, copy=True)
    for b in range(B):
        if new_done[b]:
            continue
        toks = [int(v) for v in cart[b, int(best[b]), : int(accept_len[b]) + 1]]
        c, fin = len(toks), False
        if stop_token is not None and stop_token in toks:
            c, fin = toks.index(stop_token) + 1, True
        room = min(int(max_new) - int(n_out[b]), int(Lmax) - int(seq_len[b]))
        if c >= room:
            c, fin = max(room, 0), True
        counts[b] = c
        new_done[b] = fin
    return counts, new_done


def kv_compact_counts(tree, Kc, Vc, Kt, Vt, best, counts, seq_len):
    """kv_compact with counts[b] rows (the first counts[b] nodes of the chosen path)."""
    Kc = np.array(Kc, copy=True)
    Vc = np.array(Vc, copy=True)
    seq_len = np.array(seq_len, dtype=np.int64, copy=True)
    for b in range(Kc.shape[1]):
        c = int(counts[b])
        if c == 0:
            continue
        rows = tree["retrieve"][int(best[b]), :c]
        s = int(seq_len[b])
        Kc[:, b, :, s:s + c, :] = np.asarray(Kt)[:, b][:, :, rows, :]
        Vc[:, b, :, s:s + c, :] = np.asarray(Vt)[:, b][:, :, rows, :]
        seq_len[b] = s + c
    return Kc, Vc, seq_len

