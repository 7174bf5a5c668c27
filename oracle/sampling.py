"""Sampled tokens: the root under ``sampling='typical'`` / ``'nucleus'`` and the draws
of the non-``fast`` acceptance branch.

What the pages fix ("大模型推理 memory bandwidth bound (5) - Medusa"):
* section 二.4 ``generate_candidates()``: with temperature 0 or ``fast`` the root
  is the argmax; otherwise it is one token drawn from the last logits, by
  ``get_typical_one_token(logits, temperature, posterior_threshold,
  posterior_alpha)`` or ``get_nucleus_one_token(logits, temperature, top_p)``
  (top_p defaults to 0.8 in ``medusa_generate()``, section 二.1);
* section 一.3: typical acceptance is the eta-sampling allow set
  A = {x : p(x) > eta}, eta = min(eps, delta * exp(-H(p)));
* section 二.6 ``evaluate_posterior()``: outside the ``fast`` branch a posterior
  mask comes from ``get_typical_posterior_mask(...)`` and the chosen path is the
  first one of the longest accepted length (no likelihood tie-break).

Readings where the pages stop (the bodies of those three functions are not on
the pages; parity of this module is pinned by the sampling definitions and the
invariants in ``tests/test_oracle_sampling.py``, not by the pages' code):
* q = softmax(logits / temperature).  ``typical`` draws from q restricted to
  A = {x : q(x) > eta} with eta computed exactly as in the acceptance rule
  (H = -sum q log(q + 1e-5)), renormalised; an empty A leaves the argmax.
  ``nucleus`` draws from q restricted to the smallest set of the most probable
  tokens whose mass reaches top_p (every token tied with the last one included),
  renormalised (the top-p sampling of Holtzman et al., "The Curious Case of
  Neural Text Degeneration", 2019).
* A draw is the Gumbel-max form of sampling from that renormalised
  distribution: the allowed token with the largest log q(x) + G(x),
  G(x) = -log(-log U(x)), lowest index on ties; the uniforms U come from the
  counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
  "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) keyed by the 64-bit
  seed, with counter (x // 4, position, sequence, 0) and output word x % 4 for
  token x, mapped to U = (2 * (r >> 9) + 1) / 2^24 (exact in float32, never 0
  or 1).  ``position`` is the absolute position of the token whose logits are
  sampled, so a draw depends only on (seed, sequence, position) and the logits.
* Non-fast acceptance: at every tree node one token is drawn from that node's
  logits (position = the node's position); a candidate is accepted when it
  equals the token drawn at its parent.  The next root is the token drawn at
  the selected node; after prefill the root is drawn at the last prompt position.
  With these keys the tokens appended by Medusa equal plain sampled decoding with
  the same seed, token for token -- the sampled counterpart of the greedy
  identity.

Decisions are taken in float32 like the product kernels: the allow-set test
q(x) > eta compares float32 roundings of values computed in float64.

Test infrastructure only (see ``oracle/__init__``).
"""
import numpy as np

SAMPLE_TYPICAL = 1
SAMPLE_NUCLEUS = 2

_M0, _M1 = 0xD2511F53, 0xCD9E8D57  # round multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85  # key increments (Weyl sequence)
_MASK = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds.  ctr: uint64 array [..., 4] of 32-bit words;
    key: two 32-bit words.  Returns uint64 array [..., 4] of 32-bit outputs.

    A round multiplies words 0 and 2 by the two constants (64-bit products split
    into high and low halves) and mixes: (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0);
    the key advances by the two Weyl increments before every round after the
    first."""
    c = np.array(ctr, dtype=np.uint64) & np.uint64(_MASK)
    k0, k1 = np.uint64(int(key[0]) & _MASK), np.uint64(int(key[1]) & _MASK)
    m0, m1 = np.uint64(_M0), np.uint64(_M1)
    mask = np.uint64(_MASK)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(_W0)) & mask
            k1 = (k1 + np.uint64(_W1)) & mask
        p0 = c[..., 0] * m0  # < 2^64: exact in uint64
        p1 = c[..., 2] * m1
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c = np.stack([hi1 ^ c[..., 1] ^ k0, lo1, hi0 ^ c[..., 3] ^ k1, lo0], axis=-1)
    return c


def uniforms(seed, seq, pos, V):
    """U(x) for tokens x = 0..V-1 of the draw keyed by (seed, sequence, position), float64."""
    n_words = (V + 3) // 4
    ctr = np.zeros((n_words, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(n_words, dtype=np.uint64)
    ctr[:, 1] = np.uint64(int(pos) & _MASK)
    ctr[:, 2] = np.uint64(int(seq) & _MASK)
    seed = int(seed) & ((1 << 64) - 1)
    r = philox4x32_10(ctr, (seed & _MASK, seed >> 32)).reshape(-1)[:V]
    return (2.0 * (r >> np.uint64(9)).astype(np.float64) + 1.0) / float(1 << 24)


def _q(logits_row, temperature):
    x = np.asarray(logits_row, dtype=np.float64) / temperature
    z = x - np.max(x)
    e = np.exp(z)
    return e / np.sum(e), z


def typical_allowed(logits_row, temperature, eps, delta):
    """(allowed [V] bool, q [V], eta): the eta-sampling allow set of section 一.3,
    q(x) > eta decided on float32 roundings."""
    q, _ = _q(logits_row, temperature)
    H = -np.sum(q * np.log(q + 1e-5))
    eta = min(eps, delta * np.exp(-H))
    return q.astype(np.float32) > np.float32(eta), q, eta


def nucleus_allowed(logits_row, temperature, top_p):
    """(allowed [V] bool, q [V], boundary mass gap): the smallest set of the most
    probable tokens whose mass reaches top_p, every token tied with the last one
    included.  The gap is |mass before the last included probability level - top_p|
    and |mass including it - top_p|, the smaller (a near-tie measure)."""
    q, _ = _q(logits_row, temperature)
    order = np.lexsort((np.arange(q.size), -q))  # descending, lower index first
    cs = np.cumsum(q[order])
    k = int(np.searchsorted(cs, top_p, side="left"))  # first index whose mass reaches top_p
    k = min(k, q.size - 1)
    t = q[order[k]]
    allowed = q >= t
    above = float(np.sum(q[q > t]))
    gap = min(abs(above - top_p), abs(float(np.sum(q[allowed])) - top_p))
    return allowed, q, gap


def draw(logits_row, kind, temperature, eps, delta, top_p, seed, seq, pos):
    """One sampled token.  Returns (token, info) with info = dict(allowed, score, margin):
    margin is the smallest relative distance of a decision from flipping -- the gap
    between the best and second-best allowed scores, an allow-set threshold test on a
    token that would win, or the nucleus boundary mass -- for near-tie accounting."""
    logits_row = np.asarray(logits_row, dtype=np.float64)
    V = logits_row.size
    if kind == SAMPLE_TYPICAL:
        allowed, q, eta = typical_allowed(logits_row, temperature, eps, delta)
    elif kind == SAMPLE_NUCLEUS:
        allowed, q, gap = nucleus_allowed(logits_row, temperature, top_p)
    else:
        raise ValueError("sampling kind %r" % kind)
    z = (logits_row - np.max(logits_row)) / temperature  # log q up to a constant
    u = uniforms(seed, seq, pos, V)
    g = -np.log(-np.log(u))
    score = z + g
    if not allowed.any():
        tok = int(np.argmax(logits_row))
        return tok, dict(allowed=allowed, score=score, margin=np.inf)
    s = np.where(allowed, score, -np.inf)
    tok = int(np.argmax(s))
    srt = np.sort(s[allowed])
    margins = []
    if srt.size > 1:
        margins.append((srt[-1] - srt[-2]) / max(1.0, abs(srt[-1])))
    if kind == SAMPLE_TYPICAL:
        # tokens near the threshold whose score beats the winner's could enter or leave
        rel = np.abs(q - eta) / max(eta, 1e-300)
        close = (rel < 1e-4) & (score >= s[tok] - 1e-4 * max(1.0, abs(s[tok])))
        margins += list(rel[close])
    else:
        margins.append(gap)
    return tok, dict(allowed=allowed, score=score, margin=float(min(margins)) if margins else np.inf)


def draw_rows(logits, kind, temperature, eps, delta, top_p, seed, seqs, positions):
    """draw() over rows: logits [M, V], seqs / positions [M] -> (tokens [M], margins [M])."""
    toks, margins = [], []
    for r in range(logits.shape[0]):
        t, info = draw(logits[r], kind, temperature, eps, delta, top_p, seed, seqs[r], positions[r])
        toks.append(t)
        margins.append(info["margin"])
    return np.array(toks, dtype=np.int64), np.array(margins)
