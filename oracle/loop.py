"""The whole Medusa generation loop on the oracle side.

Follows "大模型推理 memory bandwidth bound (5) - Medusa", section 二.1
``medusa_generate()``: build the tree buffers, prefill (which yields the root
token and the Medusa-head inputs), then repeat {generate candidates, tree
decoding, evaluate posterior, update inputs}.  The loop here runs a fixed number
of steps (no tokenizer or end-of-sequence token in a synthetic run) and works on
a batch of independent sequences sharing the tree.

``topk_hook(step, topk_idx, produced) -> topk_idx`` lets a test replace the
heads' top-K before candidates are built (forced-acceptance tests); ``produced``
holds, per sequence, the tokens appended so far.

Test infrastructure only (see ``oracle/__init__``).
"""
import numpy as np

from .candidates import build_candidates
from .decoder import forward, prefill
from .heads import medusa_heads_topk, root_token
from .posterior import evaluate_posterior
from .update import accepted_tokens, kv_compact


def medusa_generate(params, heads, tree, prompt, n_steps, Lmax, mode, temperature=0.0,
                    eps=0.09, delta=0.3, bf16=False, topk_hook=None):
    """Returns (tokens: list per sequence of appended tokens, per-step records)."""
    logits, h, cK, cV, seq = prefill(params, prompt, Lmax, bf16=bf16)
    B = seq.shape[0]
    root = root_token(logits[:, -1])
    h_sel = h[:, -1]
    toks = [[] for _ in range(B)]
    records = []
    for step in range(n_steps):
        topk, _ = medusa_heads_topk(h_sel, heads["W1"], heads["W2"], tree["K"], bf16=bf16)
        if topk_hook is not None:
            topk = topk_hook(step, topk, toks)
        tree_tokens, tree_pos, cart = build_candidates(tree, root, topk, seq)
        lg, hh, Kt, Vt = forward(params, tree_tokens, tree_pos, cK, cV, seq, tree["anc"], bf16=bf16)
        best, a, sel, nr, _ = evaluate_posterior(tree, lg, tree_tokens, mode, temperature, eps, delta)
        for b, t in enumerate(accepted_tokens(cart, best, a)):
            toks[b].extend(int(v) for v in t)
        cK, cV, seq = kv_compact(tree, cK, cV, Kt, Vt, best, a, seq)
        h_sel = hh[np.arange(B), sel]
        root = nr
        records.append(dict(topk=topk, tree_tokens=tree_tokens, best=best, accept_len=a, sel=sel,
                            next_root=nr))
    return toks, records
