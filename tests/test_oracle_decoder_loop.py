"""Pins of the oracle's decoder pieces, KV compaction and the whole Medusa loop (CPU).

The strongest pin is the page's lossless property under greedy acceptance: the
tokens a Medusa run appends must be exactly the tokens plain greedy decoding of
the same model produces.  Random heads are rarely right, so the forced tests
overwrite the heads' top-K with the plain-greedy continuation at chosen ranks,
which drives the accept length to 1 or 2 and exercises positions, the tree mask,
compaction and the next-root / next-heads hand-over."""
import numpy as np
import pytest

from oracle.decoder import forward, greedy_decode, prefill, rmsnorm, rope
from oracle.loop import medusa_generate
from oracle.posterior import GREEDY
from oracle.tree import tree_buffers
from oracle.update import accepted_tokens, kv_compact
from workloads import TWO_HEAD_CHOICES, TinyConfig, prompt_tokens, tiny_model


def test_rope_properties():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, 1, 16))
    k = rng.standard_normal((1, 1, 1, 16))
    np.testing.assert_allclose(rope(q, np.zeros((1, 1))), q, rtol=0, atol=0)
    for m, n, s in [(3, 1, 7), (10, 20, 100), (0, 5, 33)]:
        d1 = np.sum(rope(q, np.array([[m]])) * rope(k, np.array([[n]])))
        d2 = np.sum(rope(q, np.array([[m + s]])) * rope(k, np.array([[n + s]])))
        assert abs(d1 - d2) < 1e-12
    r = rope(q, np.array([[37]]))
    np.testing.assert_allclose(r[..., :8] ** 2 + r[..., 8:] ** 2, q[..., :8] ** 2 + q[..., 8:] ** 2, rtol=1e-12)
    # rotate-half pairs element i with i + Dh/2; at position 1 the first pair turns by 1 radian
    e = np.zeros((1, 1, 1, 16))
    e[..., 0] = 1.0
    r = rope(e, np.array([[1]]))
    assert abs(r[..., 0] - np.cos(1.0)) < 1e-15 and abs(r[..., 8] - np.sin(1.0)) < 1e-15


def test_rmsnorm_unit_rms():
    x = np.random.default_rng(1).standard_normal((4, 64)) * 7
    y = rmsnorm(x, np.ones(64), eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), 1.0, rtol=1e-14)


def test_prefill_equals_incremental_decode():
    params, _ = tiny_model(0)
    prompt = prompt_tokens(1, 2, 12, TinyConfig.vocab)
    logits, h, cK, cV, seq = prefill(params, prompt, 32)
    # incremental: feed the same tokens one by one through the cache
    from oracle.decoder import empty_cache, write_cache
    iK, iV = empty_cache(params, 2, 32)
    s = np.zeros(2, dtype=np.int64)
    one = np.ones((1, 1), bool)
    for t in range(12):
        lg, hh, Kn, Vn = forward(params, prompt[:, t:t + 1], s[:, None], iK, iV, s, one)
        write_cache(iK, iV, Kn, Vn, s)
        s = s + 1
        np.testing.assert_allclose(lg[:, 0], logits[:, t], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(hh[:, 0], h[:, t], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(iK, cK, rtol=1e-10, atol=1e-12)


def test_kv_compact_rows():
    t = tree_buffers(TWO_HEAD_CHOICES)
    rng = np.random.default_rng(2)
    Kc = rng.standard_normal((2, 2, 3, 20, 4))
    Vc = rng.standard_normal((2, 2, 3, 20, 4))
    Kt = rng.standard_normal((2, 2, 3, 9, 4))
    Vt = rng.standard_normal((2, 2, 3, 9, 4))
    best, a, seq = np.array([1, 4]), np.array([2, 0]), np.array([10, 5])
    nK, nV, ns = kv_compact(t, Kc, Vc, Kt, Vt, best, a, seq)
    assert ns.tolist() == [13, 6]
    # sequence 0: path 1 = [0, 2, 7] lands in rows 10, 11, 12
    for i, node in enumerate([0, 2, 7]):
        np.testing.assert_array_equal(nK[:, 0, :, 10 + i], Kt[:, 0, :, node])
        np.testing.assert_array_equal(nV[:, 0, :, 10 + i], Vt[:, 0, :, node])
    np.testing.assert_array_equal(nK[:, 1, :, 5], Kt[:, 1, :, 0])
    # nothing else changed
    np.testing.assert_array_equal(nK[:, 0, :, :10], Kc[:, 0, :, :10])
    np.testing.assert_array_equal(nK[:, 0, :, 13:], Kc[:, 0, :, 13:])
    np.testing.assert_array_equal(nK[:, 1, :, 6:], Kc[:, 1, :, 6:])
    cart = np.arange(2 * 6 * 3).reshape(2, 6, 3)
    assert accepted_tokens(cart, best, a) == [[3, 4, 5], [30]]


def _run(n_steps, hook=None, B=1, seed=0):
    params, heads = tiny_model(seed)
    t = tree_buffers(TWO_HEAD_CHOICES)
    prompt = prompt_tokens(seed + 100, B, TinyConfig.prompt_len, TinyConfig.vocab)
    toks, recs = medusa_generate(params, heads, t, prompt, n_steps, 160, GREEDY, topk_hook=hook)
    ref = greedy_decode(params, prompt, max(len(x) for x in toks), 160)
    return toks, recs, ref


def test_medusa_greedy_equals_plain_greedy():
    toks, recs, ref = _run(TinyConfig.n_steps, B=2)
    for b in range(2):
        assert toks[b] == ref[b, :len(toks[b])].tolist()


@pytest.mark.parametrize("ranks", [(0, 0), (1, 2), (1, None), (0, 1)])
def test_forced_acceptance_keeps_greedy_output(ranks):
    """Overwrite head 1 rank r1 (and head 2 rank r2) with the plain-greedy continuation."""
    params, heads = tiny_model(0)
    t = tree_buffers(TWO_HEAD_CHOICES)
    prompt = prompt_tokens(100, 1, TinyConfig.prompt_len, TinyConfig.vocab)
    plain = greedy_decode(params, prompt, 60, 160)[0]
    r1, r2 = ranks

    def hook(step, topk, produced):
        n = len(produced[0])  # the root of this step is plain[n]
        topk = topk.copy()
        topk[0, 0, r1] = plain[n + 1]
        if r2 is not None:
            topk[0, 1, r2] = plain[n + 2]
        return topk

    out, recs = medusa_generate(params, heads, t, prompt, 10, 160, GREEDY, topk_hook=hook)
    assert out[0] == plain[:len(out[0])].tolist()
    want = 2 if r2 is not None else 1
    assert all(int(r["accept_len"][0]) >= want for r in recs)


def _forced_two(plain):
    """Hook that makes every step accept two candidates (three tokens) per sequence."""
    def hook(step, topk, produced):
        topk = topk.copy()
        for b, prod in enumerate(produced):
            n = len(prod)
            topk[b, 0, 0] = plain[b, n + 1]
            topk[b, 1, 0] = plain[b, n + 2]
        return topk
    return hook


def test_stop_token_truncates_plain_greedy():
    """Per-sequence stop: the output is plain greedy decoding up to and including the
    first stop token (here one that falls inside a step's three accepted tokens),
    after which the sequence appends nothing and its length stays; the other
    sequence of the batch runs on to its output room."""
    params, heads = tiny_model(0)
    t = tree_buffers(TWO_HEAD_CHOICES)
    prompt = prompt_tokens(100, 2, TinyConfig.prompt_len, TinyConfig.vocab)
    plain = greedy_decode(params, prompt, 60, 160)
    k = next(i for i in range(4, 40) if i % 3 != 2 and int(plain[0, i]) not in plain[0, :i].tolist()
             and int(plain[0, i]) not in plain[1, :30].tolist())
    stop = int(plain[0, k])
    out, recs = medusa_generate(params, heads, t, prompt, 14, 160, GREEDY, topk_hook=_forced_two(plain),
                                stop_token=stop, max_new=30)
    assert out[0] == plain[0, :k + 1].tolist()
    assert out[1] == plain[1, :30].tolist()
    P = TinyConfig.prompt_len
    assert [int(r["seq_len"][0]) for r in recs][-1] == P + k + 1
    s_after = [int(r["seq_len"][0]) for r in recs if int(r["seq_len"][0]) == P + k + 1]
    assert len(s_after) >= 2  # the stopped sequence keeps its length over later steps


def test_output_room_caps_without_stop_token():
    """No stop token, max_new = 7 with three tokens accepted per step: the third
    step appends one token, and the output is the first 7 plain-greedy tokens."""
    params, heads = tiny_model(0)
    t = tree_buffers(TWO_HEAD_CHOICES)
    prompt = prompt_tokens(100, 2, TinyConfig.prompt_len, TinyConfig.vocab)
    plain = greedy_decode(params, prompt, 40, 160)
    out, recs = medusa_generate(params, heads, t, prompt, 5, 160, GREEDY, topk_hook=_forced_two(plain),
                                max_new=7)
    for b in range(2):
        assert out[b] == plain[b, :7].tolist()
    assert [int(r["counts"][0]) for r in recs] == [3, 3, 1, 0, 0]


def test_bf16_rounding_matches_torch():
    import torch
    from oracle.numerics import round_bf16
    x = np.random.default_rng(5).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0]  # exact ties round to even
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x), ref)


def test_medusa_greedy_equals_plain_greedy_bf16_points():
    params, heads = tiny_model(3)
    t = tree_buffers(TWO_HEAD_CHOICES)
    prompt = prompt_tokens(7, 1, TinyConfig.prompt_len, TinyConfig.vocab)
    plain = greedy_decode(params, prompt, 40, 160, bf16=True)[0]

    def hook(step, topk, produced):
        n = len(produced[0])
        topk = topk.copy()
        topk[0, 0, 1] = plain[n + 1]
        topk[0, 1, 0] = plain[n + 2]
        return topk

    out, recs = medusa_generate(params, heads, t, prompt, 8, 160, GREEDY, bf16=True, topk_hook=hook)
    assert out[0] == plain[:len(out[0])].tolist()
