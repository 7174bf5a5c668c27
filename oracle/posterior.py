"""Acceptance: greedy match or typical acceptance, then the longest accepted path.

Follows "大模型推理 memory bandwidth bound (5) - Medusa", section 二.6
``evaluate_posterior()`` and section 一.3 (typical acceptance):

* greedy (temperature 0): candidate token x_j on a path is accepted when it
  equals the argmax of the logits at its parent position;
* typical, ``fast`` branch: with q = softmax(logits / temperature) at the parent,
  H = -sum q log(q + 1e-5) and threshold = min(eps, delta * exp(-H)), x_j is
  accepted when q(x_j) > threshold (strict);
* the accepted length of a path is its number of leading accepted candidates;
  the step's accept length a is the maximum over paths; with a == 0 the first
  path is chosen; otherwise greedy picks the first path of length a and
  typical picks, among the paths of length a, the one with the largest
  sum of log q(x_j) over its accepted candidates (first one on a tie);
* section 二.7: the next root is the argmax at the node reached on the chosen
  path after a accepted steps, and the Medusa heads are re-applied there.

Readings where the page is silent or garbled:
* the page's parameter defaults are swapped between functions; eps is
  ``posterior_threshold`` (0.09) and delta is ``posterior_alpha`` (0.3);
* the code comment calls the threshold ``min(eps, alpha * H)``; the formula and
  the code use ``delta * exp(-H)``, which is taken;
* padded slots of ``retrieve_indices`` (-1) are never accepted (the page's
  tensor code would compare the pad token 0 against the parent's argmax);
* each decision is taken in float32, the precision of the product kernel: the
  probability and the threshold are computed in float64 and rounded to float32
  before the strict comparison.

Test infrastructure only (see ``oracle/__init__``).
"""
import numpy as np

from .numerics import argmax_first

GREEDY = 0
TYPICAL = 1


def typical_node_stats(logits_row, temperature, eps, delta):
    """(q [V], threshold) of one node's logits under typical acceptance, float64."""
    x = np.asarray(logits_row, dtype=np.float64) / temperature
    x = x - np.max(x)
    e = np.exp(x)
    q = e / np.sum(e)
    H = -np.sum(q * np.log(q + 1e-5))
    thr = min(eps, delta * np.exp(-H))
    return q, thr


def evaluate_posterior_one(tree, logits, tree_tokens, mode, temperature=0.0, eps=0.09, delta=0.3,
                           decide_dtype=np.float32, flip=()):
    """One sequence.  logits [T, V], tree_tokens [T].

    Returns dict(best, accept_len, sel, next_root, acc [P], lik [P] (typical),
    margins: list of per-decision margins used to spot near-ties, node_margin [T]:
    the relative margin |q - thr| / thr of the typical decision on each node's
    candidate, inf where none is taken).
    ``flip``: tree nodes whose accept decision is inverted -- a test hook that
    shows whether one decision lying within rounding of its threshold accounts
    for a difference from another implementation.
    """
    logits = np.asarray(logits, dtype=np.float64)
    tree_tokens = np.asarray(tree_tokens, dtype=np.int64)
    T = tree["T"]
    P, D = tree["P"], tree["D"]
    retrieve, path_len = tree["retrieve"], tree["path_len"]
    amax = argmax_first(logits, axis=-1)
    margins = []
    if mode == TYPICAL:
        if not temperature > 0:
            raise ValueError("typical acceptance needs temperature > 0")
        stats = [typical_node_stats(logits[u], temperature, eps, delta) for u in range(T)]
    acc = np.zeros(P, dtype=np.int64)
    lik = np.zeros(P, dtype=np.float64)
    node_margin = np.full(T, np.inf)
    flip = set(int(c) for c in flip)
    for p in range(P):
        n = 0
        for j in range(1, D + 1):
            if j >= path_len[p]:
                break  # padded slot: never accepted
            u = retrieve[p, j - 1]
            c = retrieve[p, j]
            tok = tree_tokens[c]
            if mode == GREEDY:
                ok = tok == amax[u]
                srt = np.sort(logits[u])
                margins.append(("argmax_gap", float(srt[-1] - srt[-2])))
            else:
                q, thr = stats[u]
                prob = q[tok]
                ok = decide_dtype(prob) > decide_dtype(thr)
                rel = float(abs(prob - thr) / max(thr, 1e-300))
                margins.append(("typical_rel", rel))
                node_margin[c] = rel
            if c in flip:
                ok = not ok
            if not ok:
                break
            n += 1
            if mode == TYPICAL:
                lik[p] += np.log(stats[u][0][tok])
        acc[p] = n
    a = int(acc.max()) if P else 0
    if a == 0:
        best = 0
    elif mode == GREEDY:
        best = int(np.flatnonzero(acc == a)[0])
    else:
        cands = np.flatnonzero(acc == a)
        best = int(cands[np.argmax(lik[cands])])
        ls = np.sort(lik[cands])
        if len(ls) > 1:
            # distinct paths with distinct accepted prefixes: their gap
            gaps = np.diff(np.unique(ls))
            margins.append(("lik_gap", float(gaps.min()) if len(gaps) else np.inf))
    sel = int(retrieve[best, a])
    next_root = int(amax[sel])
    return dict(best=best, accept_len=a, sel=sel, next_root=next_root, acc=acc, lik=lik,
                argmax=amax, margins=margins, node_margin=node_margin)


def evaluate_posterior(tree, logits, tree_tokens, mode, temperature=0.0, eps=0.09, delta=0.3):
    """Batch version: logits [B, T, V], tree_tokens [B, T] ->
    (best [B], accept_len [B], sel [B], next_root [B], per-sequence details)."""
    B = logits.shape[0]
    res = [evaluate_posterior_one(tree, logits[b], tree_tokens[b], mode, temperature, eps, delta)
           for b in range(B)]
    best = np.array([r["best"] for r in res], dtype=np.int64)
    a = np.array([r["accept_len"] for r in res], dtype=np.int64)
    sel = np.array([r["sel"] for r in res], dtype=np.int64)
    nr = np.array([r["next_root"] for r in res], dtype=np.int64)
    return best, a, sel, nr, res


def evaluate_posterior_sampled_one(tree, logits, tree_tokens, tree_pos, kind, temperature, eps=0.09, delta=0.3,
                                   top_p=0.8, seed=0, seq=0):
    """The non-``fast`` branch of section 二.6 for one sequence (the mask body is a
    reading, see ``oracle.sampling``): one token is drawn at every tree node from its
    logits (position = the node's position ``tree_pos``); a candidate is accepted when
    it equals the token drawn at its parent (pads never); the accepted length of a path
    is its number of leading accepted candidates; the chosen path is the first one of
    the longest length (path 0 when nothing is accepted); the next root is the token
    drawn at the selected node.

    Returns dict(best, accept_len, sel, next_root, acc [P], draws [T], margins [T])."""
    from .sampling import draw_rows
    logits = np.asarray(logits, dtype=np.float64)
    tree_tokens = np.asarray(tree_tokens, dtype=np.int64)
    T, P, D = tree["T"], tree["P"], tree["D"]
    retrieve, path_len = tree["retrieve"], tree["path_len"]
    draws, margins = draw_rows(logits, kind, temperature, eps, delta, top_p, seed, [seq] * T,
                               np.asarray(tree_pos, dtype=np.int64))
    acc = np.zeros(P, dtype=np.int64)
    for p in range(P):
        n = 0
        for j in range(1, D + 1):
            if j >= path_len[p]:
                break
            if tree_tokens[retrieve[p, j]] != draws[retrieve[p, j - 1]]:
                break
            n += 1
        acc[p] = n
    a = int(acc.max()) if P else 0
    best = 0 if a == 0 else int(np.flatnonzero(acc == a)[0])
    sel = int(retrieve[best, a])
    return dict(best=best, accept_len=a, sel=sel, next_root=int(draws[sel]), acc=acc, draws=draws,
                margins=margins)
