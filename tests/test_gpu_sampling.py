"""GPU parity of sampled generation (the non-fast branch) through the C ABI.

* medusa_sample_tokens draws the oracle's token on every row (typical and nucleus,
  V 512 and 32000); a differing draw is allowed only where the oracle's own
  decision sits within rounding of flipping (near-tie margin < 1e-4), counted.
* evaluate_posterior_sampled equals the oracle's non-fast rule applied to the
  GPU's own per-node draws (bit-exact), and those draws equal the oracle's up to
  counted near-ties.
* End to end on the tiny fp32 model: the tokens Medusa appends under sampled
  acceptance equal plain sampled decoding (the oracle's, and the GPU's one-node
  tree), with and without forced acceptance.
* A bf16 sampled step leaves the state the rule gives on its own logits."""
import numpy as np
import pytest

from oracle.loop import plain_sampled_decode
from oracle.posterior import evaluate_posterior_sampled_one
from oracle.sampling import SAMPLE_NUCLEUS, SAMPLE_TYPICAL, draw_rows
from oracle.tree import tree_buffers
from workloads import PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, TinyConfig, prompt_tokens, seeded_tree_choices, tiny_model

from _gpu import say, to_dev, to_np

pytestmark = pytest.mark.gpu

NEAR = 1e-4


def _sampling(kind, seed=77, tau=0.8):
    return dict(kind=kind, temperature=tau, eps=0.09, delta=0.3, top_p=0.8, seed=seed)


@pytest.mark.parametrize("kind", [SAMPLE_TYPICAL, SAMPLE_NUCLEUS])
@pytest.mark.parametrize("V,scale", [(512, 2.0), (32000, 1.0), (1001, 3.0)])
def test_sample_tokens_vs_oracle(dev, kind, V, scale):
    import torch
    from speculative_decoding_heads_amd import api
    say("sample_tokens kind", kind, "V", V)
    rng = np.random.default_rng(V + kind)
    M = 96
    lg = (rng.standard_normal((M, V)) * scale).astype(np.float32)
    pos = rng.integers(0, 100000, M).astype(np.int32)
    seq = rng.integers(0, 8, M).astype(np.int32)
    sm = _sampling(kind)
    d = lambda x: torch.from_numpy(x).to(dev)
    got = to_np(api.sample_tokens(d(lg), sm, d(pos), seq_id=d(seq)))
    torch.cuda.synchronize()
    want, margins = draw_rows(lg, kind, sm["temperature"], sm["eps"], sm["delta"], sm["top_p"], sm["seed"], seq, pos)
    diff = np.flatnonzero(got != want)
    assert all(margins[i] < NEAR for i in diff), [(int(i), int(got[i]), int(want[i]), margins[i]) for i in diff]
    assert len(diff) <= 2
    # the same rows drawn again give the same tokens (counter-based: no state)
    again = to_np(api.sample_tokens(d(lg), sm, d(pos), seq_id=d(seq)))
    assert np.array_equal(again, got)


@pytest.mark.parametrize("kind", [SAMPLE_TYPICAL, SAMPLE_NUCLEUS])
@pytest.mark.parametrize("V", [1, 2, 5])
def test_sample_tokens_tiny_vocabulary(dev, kind, V):
    """Vocabularies of 1, 2 and 5 tokens (one token: every draw is token 0)."""
    import torch
    from speculative_decoding_heads_amd import api
    say("sample_tokens tiny V", V, "kind", kind)
    rng = np.random.default_rng(7 * V + kind)
    M = 64
    lg = (rng.standard_normal((M, V)) * 1.5).astype(np.float32)
    pos = rng.integers(0, 100000, M).astype(np.int32)
    seq = rng.integers(0, 8, M).astype(np.int32)
    sm = _sampling(kind, seed=5)
    d = lambda x: torch.from_numpy(x).to(dev)
    got = to_np(api.sample_tokens(d(lg), sm, d(pos), seq_id=d(seq)))
    torch.cuda.synchronize()
    want, margins = draw_rows(lg, kind, sm["temperature"], sm["eps"], sm["delta"], sm["top_p"], sm["seed"], seq, pos)
    if V == 1:
        assert got.tolist() == [0] * M
    diff = np.flatnonzero(got != want)
    assert all(margins[i] < NEAR for i in diff), [(int(i), int(got[i]), int(want[i]), margins[i]) for i in diff]
    assert len(diff) <= 2


@pytest.mark.parametrize("kind", [SAMPLE_TYPICAL, SAMPLE_NUCLEUS])
@pytest.mark.parametrize("V,off", [(6000, 0), (12004, 0), (40000, 0), (8000, 1)])
def test_sample_tokens_row_length_variants(dev, kind, V, off):
    """Row lengths that take the draw kernel's 2- and 4-vector register sets (12004 fills the
    last set in part) and its scalar path (V > 32768, or rows whose base is not 16-byte
    aligned: ``off`` floats into the buffer)."""
    import torch
    from speculative_decoding_heads_amd import api
    say("sample_tokens kind", kind, "V", V, "offset", off)
    rng = np.random.default_rng(3 * V + kind + off)
    M = 48
    lg = (rng.standard_normal((M, V)) * 2.0).astype(np.float32)
    pos = rng.integers(0, 100000, M).astype(np.int32)
    seq = rng.integers(0, 8, M).astype(np.int32)
    sm = _sampling(kind, seed=91)
    buf = torch.empty(M * V + off, dtype=torch.float32, device=dev)
    buf[off:] = torch.from_numpy(lg.ravel()).to(dev)
    lgd = buf[off:].view(M, V)
    assert (lgd.data_ptr() % 16 != 0) == (off % 4 != 0)
    d = lambda x: torch.from_numpy(x).to(dev)
    got = to_np(api.sample_tokens(lgd, sm, d(pos), seq_id=d(seq)))
    torch.cuda.synchronize()
    want, margins = draw_rows(lg, kind, sm["temperature"], sm["eps"], sm["delta"], sm["top_p"], sm["seed"], seq, pos)
    diff = np.flatnonzero(got != want)
    assert all(margins[i] < NEAR for i in diff), [(int(i), int(got[i]), int(want[i]), margins[i]) for i in diff]
    assert len(diff) <= 2


def _node_draws(dev, lg, tree_pos, sm):
    """GPU draws at every node of every sequence (medusa_sample_tokens), [B, T]."""
    import torch
    from speculative_decoding_heads_amd import api
    B, T, V = lg.shape
    seq = np.repeat(np.arange(B, dtype=np.int32), T)
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    out = api.sample_tokens(d(lg.reshape(B * T, V)), sm, d(tree_pos.reshape(-1).astype(np.int32)), seq_id=d(seq))
    return to_np(out).reshape(B, T)


@pytest.mark.parametrize("kind", [SAMPLE_TYPICAL, SAMPLE_NUCLEUS])
@pytest.mark.parametrize("choices", [PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, seeded_tree_choices(0)])
def test_evaluate_posterior_sampled_vs_oracle(dev, kind, choices):
    import torch
    from speculative_decoding_heads_amd import api
    say("evaluate_posterior_sampled kind", kind, "T", len(choices) + 1)
    tree = api.Tree(choices)
    ot = tree_buffers(choices)
    T = ot["T"]
    rng = np.random.default_rng(T + kind)
    near = 0
    for V, scale in [(512, 2.5), (32000, 1.5)]:
        B = 4
        lg = (rng.standard_normal((B, T, V)) * scale).astype(np.float32)
        seq_len = rng.integers(100, 5000, B)
        tree_pos = (seq_len[:, None] + ot["depth"][None, :]).astype(np.int32)
        sm = _sampling(kind, seed=5 + V)
        toks = rng.integers(0, V, (B, T)).astype(np.int32)
        oracle_draws = np.zeros((B, T), np.int64)
        for b in range(B):
            dr, _ = draw_rows(lg[b], kind, sm["temperature"], sm["eps"], sm["delta"], sm["top_p"], sm["seed"],
                              [b] * T, tree_pos[b])
            oracle_draws[b] = dr
            for c in range(1, T):  # make most candidates equal their parent's draw
                if rng.uniform() < 0.75:
                    toks[b, c] = dr[ot["parent"][c]]
        d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        outs = api.evaluate_posterior_sampled(tree, d(lg), d(toks), d(tree_pos), sm)
        gdraws = _node_draws(dev, lg, tree_pos, sm)
        torch.cuda.synchronize()
        got = np.stack([to_np(x) for x in outs], 1)
        for b in range(B):
            r = evaluate_posterior_sampled_one(ot, lg[b], toks[b], tree_pos[b], kind, sm["temperature"], sm["eps"],
                                               sm["delta"], sm["top_p"], sm["seed"], b)
            for u in np.flatnonzero(gdraws[b] != r["draws"]):
                assert r["margins"][u] < NEAR, (b, int(u), int(gdraws[b, u]), int(r["draws"][u]))
                near += 1
            # the rule on the GPU's own draws: bit-exact
            acc = []
            for p in range(ot["P"]):
                n = 0
                for j in range(1, int(ot["path_len"][p])):
                    if toks[b, ot["retrieve"][p, j]] != gdraws[b, ot["retrieve"][p, j - 1]]:
                        break
                    n += 1
                acc.append(n)
            a = max(acc)
            best = 0 if a == 0 else acc.index(a)
            sel = int(ot["retrieve"][best, a])
            assert tuple(got[b]) == (best, a, sel, int(gdraws[b, sel])), (b, got[b])
            if np.array_equal(gdraws[b], r["draws"]):
                assert tuple(got[b]) == (r["best"], r["accept_len"], r["sel"], r["next_root"])
    assert near <= 3


def _upload(params, heads, dev):
    import torch
    P = dict(params)
    for k in ("embed", "final_norm", "lm_head"):
        P[k] = to_dev(params[k], torch.float32, dev)
    P["layers"] = [{k: to_dev(v, torch.float32, dev) for k, v in l.items()} for l in params["layers"]]
    return P, {k: to_dev(v, torch.float32, dev) for k, v in heads.items()}


def _gpu_sampled_run(dev, params, heads, choices, prompt, n_steps, sm, override=None):
    import torch
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import SAMPLED
    from speculative_decoding_heads_amd.model import Model, State, prefill, step
    P, H = _upload(params, heads, dev)
    model = Model(P, H, max_pos=1024)
    tree = api.Tree(choices)
    B = prompt.shape[0]
    st = State(model, B, 256, 128, sampling=sm)
    prefill(model, st, torch.from_numpy(prompt.astype(np.int32)).to(dev))
    accs = []
    for s in range(n_steps):
        ov = None
        if override is not None:
            ov = torch.from_numpy(override(to_np(st.n_out)).astype(np.int32)).to(dev)
        step(model, tree, st, SAMPLED, L_hint=256, topk_override=ov)
        accs.append(to_np(st.accept_len).copy())
    torch.cuda.synchronize()
    assert int(to_np(st.err)[0]) == 0
    n, toks = to_np(st.n_out), to_np(st.out_tokens)
    return [toks[b, : n[b]].tolist() for b in range(B)], accs


@pytest.mark.parametrize("kind", [SAMPLE_TYPICAL, SAMPLE_NUCLEUS])
@pytest.mark.parametrize("forced", [False, True])
def test_tiny_fp32_sampled_medusa_equals_plain_sampled_decoding(dev, kind, forced):
    say("e2e tiny fp32 sampled medusa kind", kind, "forced", forced)
    params, heads = tiny_model(0)
    prompt = prompt_tokens(100, 2, TinyConfig.prompt_len, TinyConfig.vocab)
    sm = _sampling(kind, seed=2024)
    plain = plain_sampled_decode(params, prompt, 60, 256, sm)
    override = None
    if forced:
        def override(n_out):
            ov = np.zeros((2, 2, 3), np.int64)
            for b in range(2):
                n = int(n_out[b])
                ov[b] = (plain[b, n + 1] + 1 + np.arange(6).reshape(2, 3)) % TinyConfig.vocab
                ov[b, 0, 1] = plain[b, n + 1]
                ov[b, 1, 0] = plain[b, n + 2]
            return ov
    med, accs = _gpu_sampled_run(dev, params, heads, TWO_HEAD_CHOICES, prompt, 12, sm, override)
    one, _ = _gpu_sampled_run(dev, params, heads, [], prompt, max(len(m) for m in med), sm)
    for b in range(2):
        assert med[b] == plain[b, : len(med[b])].tolist(), "GPU sampled medusa != plain sampled decoding"
        assert one[b] == plain[b, : len(one[b])].tolist(), "GPU one-node sampled decoding != oracle"
    if forced:
        assert all((a == 2).all() for a in accs)


def _gpu_sampled_fused_run(dev, params, heads, choices, prompt, n_steps, sm):
    """As _gpu_sampled_run, with the fused draft + verify step (heads on every node)."""
    import torch
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import SAMPLED
    from speculative_decoding_heads_amd.model import Model, State, init_topk_carry, prefill, step_fused
    P, H = _upload(params, heads, dev)
    model = Model(P, H, max_pos=1024)
    tree = api.Tree(choices)
    B = prompt.shape[0]
    st = State(model, B, 256, 128, sampling=sm)
    prefill(model, st, torch.from_numpy(prompt.astype(np.int32)).to(dev))
    carry = init_topk_carry(model, tree, st)
    accs = []
    for s in range(n_steps):
        step_fused(model, tree, st, carry, SAMPLED, L_hint=256)
        accs.append(to_np(st.accept_len).copy())
    torch.cuda.synchronize()
    assert int(to_np(st.err)[0]) == 0
    n, toks = to_np(st.n_out), to_np(st.out_tokens)
    return [toks[b, : n[b]].tolist() for b in range(B)], accs


@pytest.mark.parametrize("kind", [SAMPLE_TYPICAL, SAMPLE_NUCLEUS])
def test_tiny_fp32_fused_sampled_equals_step(dev, kind):
    """The fused draft + verify step with sampled acceptance: the fp32 heads give the
    same top-K on every node as on the selected node alone, and the draws depend only
    on (sequence, position), so tokens and per-step accepted lengths equal the plain
    step's, and the tokens equal plain sampled decoding in the oracle."""
    say("e2e tiny fp32 fused sampled kind", kind)
    params, heads = tiny_model(0)
    prompt = prompt_tokens(101, 2, TinyConfig.prompt_len, TinyConfig.vocab)
    sm = _sampling(kind, seed=77)
    fused, facc = _gpu_sampled_fused_run(dev, params, heads, TWO_HEAD_CHOICES, prompt, 10, sm)
    plain_step, pacc = _gpu_sampled_run(dev, params, heads, TWO_HEAD_CHOICES, prompt, 10, sm)
    assert fused == plain_step
    assert all(np.array_equal(a, b) for a, b in zip(facc, pacc))
    ref = plain_sampled_decode(params, prompt, max(len(f) for f in fused) + 1, 256, sm)
    for b in range(2):
        assert fused[b] == ref[b, : len(fused[b])].tolist(), "fused sampled medusa != plain sampled decoding"


def test_bf16_sampled_step_state(dev):
    """A bf16 sampled step (page tree, typical draws) leaves the state the non-fast
    rule gives on the same forward's logits: acceptance, compaction, next root."""
    import torch
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import SAMPLED
    from speculative_decoding_heads_amd.model import Model, State, prefill, step
    say("e2e bf16 sampled step")

    class Cfg:
        n_layers = 2
        d = 512
        n_heads, n_kv_heads, head_dim = 8, 4, 64
        ffn = 1024
        vocab = 2048
        n_medusa = 4
        rope_theta = 10000.0
        norm_eps = 1e-6
    params, heads = tiny_model(5, cfg=Cfg, bf16=True)
    P = dict(params)
    for k in ("embed", "final_norm", "lm_head"):
        P[k] = to_dev(params[k], torch.bfloat16, dev)
    P["layers"] = [{k: to_dev(v, torch.bfloat16, dev) for k, v in l.items()} for l in params["layers"]]
    model = Model(P, {k: to_dev(v, torch.bfloat16, dev) for k, v in heads.items()}, max_pos=1024)
    tree = api.Tree(PAGE_TREE_CHOICES)
    ot = tree_buffers(PAGE_TREE_CHOICES)
    B, Lmax = 2, 256
    sm = _sampling(SAMPLE_TYPICAL, seed=11, tau=1.0)
    st = State(model, B, Lmax, 64, sampling=sm)
    prefill(model, st, torch.from_numpy(prompt_tokens(9, B, 70, Cfg.vocab).astype(np.int32)).to(dev))
    root, seq0, h0 = st.root.clone(), st.seq_len.clone(), st.h_sel.clone()
    Kc0, Vc0 = st.Kc.clone(), st.Vc.clone()
    step(model, tree, st, SAMPLED, L_hint=Lmax)
    topk, _ = api.medusa_heads_topk(h0, model.W1, model.W2, tree.K)
    tok, pos, cart = api.tree_build_candidates(tree, root, topk, seq0)
    logits, h, Kt, Vt = model.forward(tok, pos, Kc0, Vc0, seq0, tree, L_hint=Lmax)
    ref = api.evaluate_posterior_sampled(tree, logits, tok, pos, sm)
    torch.cuda.synchronize()
    for name, r in zip(("best", "accept_len", "sel_node", "root"), ref):
        assert torch.equal(getattr(st, name), r), name
    for b in range(B):
        a, bi = int(st.accept_len[b]), int(st.best[b])
        s0 = int(seq0[b])
        rows = ot["retrieve"][bi, : a + 1]
        assert torch.equal(st.Kc[:, b, :, s0:s0 + a + 1], Kt[:, b][:, :, rows])
        assert int(st.seq_len[b]) == s0 + a + 1
        assert torch.equal(st.h_sel[b], h[b, int(st.sel_node[b])])
