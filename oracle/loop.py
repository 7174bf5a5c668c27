"""The whole Medusa generation loop on the oracle side.

Follows "大模型推理 memory bandwidth bound (5) - Medusa", section 二.1
``medusa_generate()``: build the tree buffers, prefill (which yields the root
token and the Medusa-head inputs), then repeat {generate candidates, tree
decoding, evaluate posterior, update inputs}.  The loop here runs a fixed number
of steps (no tokenizer or end-of-sequence token in a synthetic run) and works on
a batch of independent sequences sharing the tree.  With ``stop_token`` (and/or
``max_new``) each sequence stops on its own: it appends up to and including the
first stop token, or until its output or cache room is used, and then appends
nothing more (``update.appended_counts``).

``topk_hook(step, topk_idx, produced) -> topk_idx`` lets a test replace the
heads' top-K before candidates are built (forced-acceptance tests); ``produced``
holds, per sequence, the tokens appended so far.

Test infrastructure only (see ``oracle/__init__``).
"""
import numpy as np

from .candidates import build_candidates
from .decoder import forward, prefill, write_cache
from .heads import medusa_heads_topk, root_token
from .posterior import evaluate_posterior, evaluate_posterior_sampled_one
from .sampling import draw
from .update import accepted_tokens, appended_counts, kv_compact, kv_compact_counts


def _draw_last(logits, sampling, seq_positions):
    """The sampled root of every sequence from its last logits (position seq_positions[b])."""
    s = sampling
    return np.array([draw(logits[b], s["kind"], s["temperature"], s["eps"], s["delta"], s["top_p"], s["seed"], b,
                          int(seq_positions[b]))[0] for b in range(logits.shape[0])], dtype=np.int64)


def medusa_generate(params, heads, tree, prompt, n_steps, Lmax, mode, temperature=0.0,
                    eps=0.09, delta=0.3, bf16=False, topk_hook=None, stop_token=None, max_new=None,
                    sampling=None):
    """Returns (tokens: list per sequence of appended tokens, per-step records).

    ``sampling`` (dict kind, temperature, eps, delta, top_p, seed) selects the
    non-``fast`` branch: sampled root and draw-matching acceptance (``mode`` ignored)."""
    logits, h, cK, cV, seq = prefill(params, prompt, Lmax, bf16=bf16)
    B = seq.shape[0]
    root = root_token(logits[:, -1]) if sampling is None else _draw_last(logits[:, -1], sampling, seq - 1)
    h_sel = h[:, -1]
    toks = [[] for _ in range(B)]
    done = np.zeros(B, dtype=bool)
    records = []
    for step in range(n_steps):
        topk, _ = medusa_heads_topk(h_sel, heads["W1"], heads["W2"], tree["K"], bf16=bf16)
        if topk_hook is not None:
            topk = topk_hook(step, topk, toks)
        tree_tokens, tree_pos, cart = build_candidates(tree, root, topk, seq)
        lg, hh, Kt, Vt = forward(params, tree_tokens, tree_pos, cK, cV, seq, tree["anc"], bf16=bf16)
        if sampling is None:
            best, a, sel, nr, _ = evaluate_posterior(tree, lg, tree_tokens, mode, temperature, eps, delta)
        else:
            sm = sampling
            rs = [evaluate_posterior_sampled_one(tree, lg[b], tree_tokens[b], tree_pos[b], sm["kind"],
                                                 sm["temperature"], sm["eps"], sm["delta"], sm["top_p"], sm["seed"], b)
                  for b in range(B)]
            best, a, sel, nr = (np.array([r[k] for r in rs], dtype=np.int64)
                                for k in ("best", "accept_len", "sel", "next_root"))
        counts = None
        if stop_token is None and max_new is None:
            for b, t in enumerate(accepted_tokens(cart, best, a)):
                toks[b].extend(int(v) for v in t)
            cK, cV, seq = kv_compact(tree, cK, cV, Kt, Vt, best, a, seq)
        else:
            n_out = np.array([len(t) for t in toks])
            counts, done = appended_counts(cart, best, a, stop_token, done, n_out,
                                           max_new if max_new is not None else 1 << 30, seq, Lmax)
            for b in range(B):
                toks[b].extend(int(v) for v in cart[b, int(best[b]), : int(counts[b])])
            cK, cV, seq = kv_compact_counts(tree, cK, cV, Kt, Vt, best, counts, seq)
        h_sel = hh[np.arange(B), sel]
        root = nr
        records.append(dict(topk=topk, tree_tokens=tree_tokens, best=best, accept_len=a, sel=sel,
                            next_root=nr, counts=counts, seq_len=np.array(seq, copy=True)))
    return toks, records


def plain_sampled_decode(params, prompt, n_new, Lmax, sampling, bf16=False):
    """Plain autoregressive sampled decoding, one token per forward: the token at
    position p + 1 is drawn from the logits at position p with the draw keyed by
    (seed, sequence, p) -- the baseline the sampled Medusa loop must reproduce.
    Returns [B, n_new]."""
    logits, h, cK, cV, seq = prefill(params, prompt, Lmax, bf16=bf16)
    tok = _draw_last(logits[:, -1], sampling, seq - 1)
    out = [tok]
    one = np.ones((1, 1), dtype=bool)
    for _ in range(n_new - 1):
        logits, h, Kn, Vn = forward(params, tok[:, None], seq[:, None], cK, cV, seq, one, bf16=bf16)
        write_cache(cK, cV, Kn, Vn, seq)
        tok = _draw_last(logits[:, -1], sampling, seq)
        seq = seq + 1
        out.append(tok)
    return np.stack(out, axis=1)
