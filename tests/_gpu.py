"""Helpers shared by the GPU parity tests (not collected)."""
import sys

import numpy as np


def say(*a):
    """Name the case before a GPU step, flushed, so a failing run shows where it was."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dtype).contiguous()


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def assert_close(got, ref, rtol, atol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), what + ": non-finite output"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError("%s: %d/%d elements out of tolerance; worst at %s got %r ref %r" %
                             (what, int(bad.sum()), bad.size, i, got[i], ref[i]))


def anc_tensor(anc_bool, dev):
    """Pack an oracle [T, T] bool mask into device int64 words (bit j = column j)."""
    import torch
    a = np.asarray(anc_bool, dtype=bool)
    words = np.zeros(a.shape[0], dtype=np.uint64)
    for i in range(a.shape[0]):
        for j in np.flatnonzero(a[i]):
            words[i] |= np.uint64(1) << np.uint64(j)
    return torch.from_numpy(words.view(np.int64)).to(dev)


def posterior_outcome(ot, logits, toks, mode, tau, eps, delta, got, rel=1e-5):
    """Compare a GPU acceptance outcome (best, accept_len, sel, next_root) with the oracle's
    on the same logits.  Returns 0 when they are equal, 1 when they differ only through
    one near-tied typical decision: either inverting the oracle's decision on a single
    node whose probability lies within ``rel`` (relative) of its threshold reproduces the
    GPU outcome exactly, or the GPU chose another longest path whose log-likelihood is
    within 1e-6 (relative) of the oracle's best.  Anything else fails.  Greedy decisions
    compare identical float32 logits and get no excuse."""
    from oracle.posterior import TYPICAL, evaluate_posterior_one
    got = tuple(int(x) for x in got)
    r = evaluate_posterior_one(ot, logits, toks, mode, tau, eps, delta)
    ref = (r["best"], r["accept_len"], r["sel"], r["next_root"])
    if got == ref:
        return 0
    if mode == TYPICAL:
        for c in np.flatnonzero(r["node_margin"] < rel):
            r2 = evaluate_posterior_one(ot, logits, toks, mode, tau, eps, delta, flip={int(c)})
            if (r2["best"], r2["accept_len"], r2["sel"], r2["next_root"]) == got:
                return 1
        gb, ga = got[0], got[1]
        if ga == r["accept_len"] and ga > 0 and 0 <= gb < len(r["acc"]) and r["acc"][gb] == ga:
            lb, lr = r["lik"][gb], r["lik"][r["best"]]
            sel = int(ot["retrieve"][gb, ga])
            if abs(lb - lr) <= 1e-6 * max(1.0, abs(lr)) and got[2] == sel and got[3] == int(r["argmax"][sel]):
                return 1
    raise AssertionError("acceptance mismatch: GPU %s, oracle %s (no single near-tied decision explains it)"
                         % (got, ref))


def check_heads_topk(gi, gv, ref_logits):
    """Logits at the returned indices match the oracle; indices bit-exact except
    where the oracle's own ranking has a near-tie at the measured error level."""
    from oracle.heads import topk_desc
    ref_idx = topk_desc(ref_logits, 10)
    B, H = ref_logits.shape[:2]
    err = 0.0
    for b in range(B):
        for k in range(H):
            rl = ref_logits[b, k]
            assert_close(gv[b, k], rl[gi[b, k]], rtol=2e-2, atol=1e-2, what="topk values")
            err = max(err, float(np.abs(gv[b, k] - rl[gi[b, k]]).max()))
    mism = 0
    for b in range(B):
        for k in range(H):
            if gi[b, k].tolist() != ref_idx[b, k].tolist():
                # allowed only where the reference ranking has a gap below the measured error
                kth = np.sort(ref_logits[b, k])[::-1]
                gap = np.min(np.abs(np.diff(kth[:11])))
                assert gap <= 4 * err + 1e-7, "top-K mismatch without near-tie (b=%d k=%d)" % (b, k)
                mism += 1
    assert mism <= max(B, 1)


def layer_stage_parity(params, p, l, tr, cK, cV, gK, gV, pos, seq, anc, rtol=2e-2, atol=1e-2):
    """Every stage of decoder layer l against the oracle's stage fed the GPU's own input
    to that stage (the buffers of medusa_forward_trace, as float64 arrays in tr):
    attention RMSNorm, rotated q and tree K/V, tree attention, the attention block's
    residual, the SwiGLU product and the layer's output stream.  Returns the largest
    absolute difference seen."""
    from oracle.attention import tree_attention
    from oracle.decoder import attention_residual, down_residual, ffn_act, qkv_rotary, rmsnorm
    from oracle.numerics import round_bf16
    B, T = pos.shape
    Hq, Dh = params["n_heads"], params["head_dim"]
    tol = dict(rtol=rtol, atol=atol)
    shape = lambda a: a.reshape(B, T, -1)
    x_in, xn, x_mid = shape(tr["x"][l]), shape(tr["xn"][l]), shape(tr["x_mid"][l])
    q = tr["q"][l].reshape(B, T, Hq, Dh)
    att = tr["attn"][l].reshape(B, T, Hq, Dh)
    worst = 0.0

    def cmp(got, ref, what):
        nonlocal worst
        assert_close(got, ref, what="layer %d %s" % (l, what), **tol)
        worst = max(worst, float(np.abs(np.asarray(got, np.float64) - ref).max()))

    cmp(xn, round_bf16(rmsnorm(x_in, p["attn_norm"], params["norm_eps"])), "attention norm")
    q_o, K_o, V_o = qkv_rotary(params, p, xn, pos, bf16=True)
    cmp(q, q_o, "rotated q")
    cmp(gK, K_o, "tree K")
    cmp(gV, V_o, "tree V")
    cmp(att, round_bf16(tree_attention(q, cK, cV, seq, gK, gV, anc, 1.0 / np.sqrt(Dh))), "tree attention")
    cmp(x_mid, attention_residual(p, x_in, att, bf16=True), "attention residual")
    act = shape(tr["act"][l])
    cmp(act, ffn_act(params, p, x_mid, bf16=True), "SwiGLU product")
    cmp(shape(tr["x"][l + 1]), down_residual(p, x_mid, act, bf16=True), "down residual")
    return worst
