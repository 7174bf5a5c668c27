"""Pins of the oracle's sampling (CPU): the counter-based generator against its
published known-answer vectors, the uniform mapping, the sampled distribution
against the renormalised truncated distribution it defines (chi-square), the
nucleus set against a brute-force enumeration, special cases that reduce to the
argmax or to the full softmax, the non-fast acceptance at vanishing temperature
against the greedy rule, and the sampled Medusa loop against plain sampled
decoding token for token (with and without forced acceptance)."""
import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle.loop import medusa_generate, plain_sampled_decode
from oracle.posterior import GREEDY, evaluate_posterior_one, evaluate_posterior_sampled_one
from oracle.sampling import (SAMPLE_NUCLEUS, SAMPLE_TYPICAL, draw, nucleus_allowed, philox4x32_10,
                             typical_allowed, uniforms)
from oracle.tree import tree_buffers
from workloads import PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, TinyConfig, prompt_tokens, tiny_model

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        ctr = np.array([int(x, 16) for x in v["ctr"]], dtype=np.uint64)
        key = [int(x, 16) for x in v["key"]]
        out = philox4x32_10(ctr, key)
        assert ["%08x" % int(x) for x in out] == v["out"]


def test_uniforms_open_interval_float32_exact_and_mean():
    u = uniforms(seed=7, seq=3, pos=11, V=100003)
    assert u.min() > 0.0 and u.max() < 1.0
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    assert abs(u.mean() - 0.5) < 0.005
    # distinct keys give distinct streams; the same key repeats exactly
    assert not np.array_equal(u[:1000], uniforms(7, 3, 12, 1000))
    assert not np.array_equal(u[:1000], uniforms(7, 4, 11, 1000))
    assert np.array_equal(u[:1000], uniforms(7, 3, 11, 1000))
    # counter word x // 4, output word x % 4
    r = philox4x32_10(np.array([2, 11, 3, 0], dtype=np.uint64), (7, 0))
    assert u[9] == (2.0 * float(int(r[1]) >> 9) + 1.0) / (1 << 24)


def _renormalised(q, allowed):
    w = np.where(allowed, q, 0.0)
    return w / w.sum()


@pytest.mark.parametrize("kind", [SAMPLE_TYPICAL, SAMPLE_NUCLEUS])
def test_draw_frequencies_match_the_truncated_distribution(kind):
    """20000 draws (distinct positions) from fixed logits: chi-square against the
    renormalised truncated distribution; excluded tokens never drawn."""
    logits = np.array([2.0, 1.5, 1.0, 0.2, -0.5, -3.0, -4.0, 1.2])
    tau, eps, delta, top_p = 0.9, 0.09, 0.3, 0.8
    if kind == SAMPLE_TYPICAL:
        allowed, q, _ = typical_allowed(logits, tau, eps, delta)
    else:
        allowed, q, _ = nucleus_allowed(logits, tau, top_p)
    assert 1 < allowed.sum() < logits.size  # a real truncation
    p = _renormalised(q, allowed)
    n = 20000
    toks = np.array([draw(logits, kind, tau, eps, delta, top_p, 99, 0, pos)[0] for pos in range(n)])
    counts = np.bincount(toks, minlength=logits.size)
    assert counts[~allowed].sum() == 0
    obs, exp = counts[allowed], n * p[allowed]
    assert stats.chisquare(obs, exp).pvalue > 1e-4


def test_nucleus_set_equals_brute_force_minimal_top_set():
    rng = np.random.default_rng(3)
    for trial in range(200):
        V = int(rng.integers(2, 12))
        logits = rng.standard_normal(V) * 2
        top_p = float(rng.uniform(0.05, 0.99))
        allowed, q, _ = nucleus_allowed(logits, 1.0, top_p)
        # brute force: the smallest k such that the k most probable tokens reach top_p
        order = np.argsort(-q, kind="stable")
        k = next(k for k in range(1, V + 1) if q[order[:k]].sum() >= top_p)
        want = np.zeros(V, bool)
        want[order[:k]] = True
        assert np.array_equal(allowed, want), (trial, q, top_p)


def test_special_cases_reduce_to_argmax_or_full_softmax():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal(50) * 2
    amax = int(np.argmax(logits))
    # top_p -> 0: the nucleus is the most probable token alone
    for pos in range(50):
        assert draw(logits, SAMPLE_NUCLEUS, 0.7, 0.09, 0.3, 1e-9, 1, 0, pos)[0] == amax
    # eps = 0: eta = 0, every token allowed (the full softmax); top_p = 1 likewise
    assert typical_allowed(logits, 0.7, 0.0, 0.3)[0].all()
    assert nucleus_allowed(logits, 0.7, 1.0)[0].all()
    # eps >= 1 and delta * exp(-H) >= 1: eta >= 1 exceeds every q, empty set -> argmax
    allowed, q, eta = typical_allowed(logits, 0.7, 2.0, 1e9)
    assert eta >= 1.0 and not allowed.any()
    assert all(draw(logits, SAMPLE_TYPICAL, 0.7, 2.0, 1e9, 0.8, 1, 0, pos)[0] == amax for pos in range(20))
    # vanishing temperature: all the mass on the argmax, both kinds draw it
    for kind in (SAMPLE_TYPICAL, SAMPLE_NUCLEUS):
        assert all(draw(logits, kind, 1e-4, 0.09, 0.3, 0.8, 1, 0, pos)[0] == amax for pos in range(20))


def test_non_fast_acceptance_at_vanishing_temperature_is_greedy():
    rng = np.random.default_rng(8)
    for choices in (PAGE_TREE_CHOICES, TWO_HEAD_CHOICES):
        t = tree_buffers(choices)
        T = t["T"]
        for trial in range(10):
            lg = rng.standard_normal((T, 40)) * 3
            toks = rng.integers(0, 40, T)
            amax = lg.argmax(1)
            for c in range(1, T):
                if rng.uniform() < 0.7:
                    toks[c] = amax[t["parent"][c]]
            pos = 100 + t["depth"]
            g = evaluate_posterior_one(t, lg, toks, GREEDY)
            for kind in (SAMPLE_TYPICAL, SAMPLE_NUCLEUS):
                s = evaluate_posterior_sampled_one(t, lg, toks, pos, kind, 1e-4, seed=3, seq=0)
                assert (s["best"], s["accept_len"], s["sel"], s["next_root"]) == \
                    (g["best"], g["accept_len"], g["sel"], g["next_root"])


@pytest.mark.parametrize("kind", [SAMPLE_TYPICAL, SAMPLE_NUCLEUS])
@pytest.mark.parametrize("forced", [False, True])
def test_sampled_medusa_equals_plain_sampled_decoding(kind, forced):
    """The tokens Medusa appends under the non-fast branch are those of plain sampled
    decoding with the same seed; with the heads' candidates replaced by the plain
    continuation (head 1 rank 1, head 2 rank 0) every step accepts two tokens."""
    params, heads = tiny_model(0)
    prompt = prompt_tokens(100, 2, TinyConfig.prompt_len, TinyConfig.vocab)
    sm = dict(kind=kind, temperature=0.8, eps=0.09, delta=0.3, top_p=0.8, seed=2024)
    tree = tree_buffers(TWO_HEAD_CHOICES)
    plain = plain_sampled_decode(params, prompt, 50, 256, sm)
    hook = None
    if forced:
        def hook(step, topk, produced):
            ov = np.array(topk, copy=True)
            for b in range(2):
                n = len(produced[b])
                ov[b, 0, 1] = plain[b, n + 1]
                ov[b, 1, 0] = plain[b, n + 2]
            return ov
    med, recs = medusa_generate(params, heads, tree, prompt, 12, 256, GREEDY, topk_hook=hook, sampling=sm)
    for b in range(2):
        assert med[b] == plain[b, : len(med[b])].tolist()
    if forced:
        assert all((r["accept_len"] == 2).all() for r in recs)
