"""GPU parity of the other verify-step calls against the oracle: candidates,
acceptance, KV compaction, Medusa heads + top-K, and the product epilogues.

Integer outputs (indices, accept lengths, tokens, copied rows) must be bit-exact.
Acceptance is checked on identical logits; the typical rule takes its decisions
in float32 on both sides and a decision whose probability lies within 1e-5
(relative) of its threshold may go either way (such near-ties are counted)."""
import numpy as np
import pytest

from oracle.candidates import build_candidates
from oracle.heads import medusa_heads_logits, topk_desc
from oracle.numerics import silu
from oracle.posterior import GREEDY, TYPICAL, evaluate_posterior_one
from oracle.tree import tree_buffers
from oracle.update import kv_compact as oracle_compact
from workloads import PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, heads_weights, seeded_tree_choices

from _gpu import assert_close, check_heads_topk, posterior_outcome, say, to_dev, to_np

pytestmark = pytest.mark.gpu

TREES = [PAGE_TREE_CHOICES, seeded_tree_choices(0), TWO_HEAD_CHOICES, [(0,), (1,), (0, 0)]]


@pytest.mark.parametrize("ti", range(len(TREES)))
def test_candidates_bit_exact(dev, ti):
    import torch
    from speculative_decoding_heads_amd import api
    choices = TREES[ti]
    say("tree_build_candidates tree", ti)
    tree = api.Tree(choices)
    ot = tree_buffers(choices)
    rng = np.random.default_rng(ti)
    B, H = 5, ot["D"] + 1
    root = rng.integers(0, 32000, B).astype(np.int32)
    topk = rng.integers(0, 32000, (B, H, ot["K"])).astype(np.int32)
    seq = rng.integers(0, 5000, B).astype(np.int32)
    d = lambda x: torch.from_numpy(x).to(dev)
    tok, pos, cart = api.tree_build_candidates(tree, d(root), d(topk), d(seq))
    torch.cuda.synchronize()
    rt, rp, rc = build_candidates(ot, root, topk, seq)
    assert np.array_equal(to_np(tok), rt) and np.array_equal(to_np(pos), rp) and np.array_equal(to_np(cart), rc)


def _posterior_case(rng, ot, B, V, mode, match_p=0.7, scale=3.0):
    T = ot["T"]
    lg = (rng.standard_normal((B, T, V)) * scale).astype(np.float32)
    toks = rng.integers(0, V, (B, T)).astype(np.int32)
    for b in range(B):
        amax = lg[b].argmax(1)
        for c in range(1, T):
            if rng.uniform() < match_p:
                toks[b, c] = amax[ot["parent"][c]]
    return lg, toks


@pytest.mark.parametrize("ti", range(len(TREES)))
@pytest.mark.parametrize("mode", [GREEDY, TYPICAL])
def test_posterior_bit_exact(dev, ti, mode):
    import torch
    from speculative_decoding_heads_amd import api
    choices = TREES[ti]
    tree = api.Tree(choices)
    ot = tree_buffers(choices)
    rng = np.random.default_rng(100 + ti + 10 * mode)
    near = 0
    for V, scale in [(512, 3.0), (32000, 1.0)]:
        say("evaluate_posterior tree", ti, "mode", mode, "V", V)
        B = 6
        lg, toks = _posterior_case(rng, ot, B, V, mode, scale=scale)
        tau, eps, delta = 0.7, 0.09, 0.3
        best, a, sel, nr = api.evaluate_posterior(tree, torch.from_numpy(lg).to(dev), torch.from_numpy(toks).to(dev),
                                                  mode, tau, eps, delta)
        torch.cuda.synchronize()
        got = np.stack([to_np(x) for x in (best, a, sel, nr)], 1)
        for b in range(B):
            near += posterior_outcome(ot, lg[b], toks[b], mode, tau, eps, delta, got[b])
    assert near <= 1


def test_posterior_typical_extremes(dev):
    """eps = 0 accepts every candidate; a threshold above 1 accepts none (special cases of the rule)."""
    import torch
    from speculative_decoding_heads_amd import api
    say("evaluate_posterior extremes")
    ot = tree_buffers(PAGE_TREE_CHOICES)
    tree = api.Tree(PAGE_TREE_CHOICES)
    rng = np.random.default_rng(7)
    lg = rng.standard_normal((2, 64, 1000)).astype(np.float32)
    toks = rng.integers(0, 1000, (2, 64)).astype(np.int32)
    d = lambda x: torch.from_numpy(x).to(dev)
    best, a, sel, nr = api.evaluate_posterior(tree, d(lg), d(toks), TYPICAL, 0.7, 0.0, 0.3)
    torch.cuda.synchronize()
    assert to_np(a).tolist() == [4, 4]
    for b in range(2):
        r = evaluate_posterior_one(ot, lg[b], toks[b], TYPICAL, 0.7, 0.0, 0.3)
        assert (int(to_np(best)[b]), int(to_np(sel)[b])) == (r["best"], r["sel"])
    best, a, sel, nr = api.evaluate_posterior(tree, d(lg), d(toks), TYPICAL, 0.7, 2.0, 1e6)
    torch.cuda.synchronize()
    assert to_np(a).tolist() == [0, 0] and to_np(best).tolist() == [0, 0] and to_np(sel).tolist() == [0, 0]
    assert to_np(nr).tolist() == lg[:, 0].argmax(1).tolist()


@pytest.mark.parametrize("V,off", [(6000, 0), (12004, 0), (16388, 0), (32001, 0), (40000, 0), (8000, 1)])
@pytest.mark.parametrize("mode", [GREEDY, TYPICAL])
def test_posterior_row_length_variants(dev, V, off, mode):
    """Row lengths that take each register-set size of the per-node statistics (1024 threads
    holding 1, 2, 4 or 8 four-float vectors; V 6000, 12004 and 16388 fill the last set only in
    part) and the scalar path (V % 4 != 0, V > 32768, or a row base that is not 16-byte
    aligned: ``off`` floats into the buffer).  Greedy: every candidate is its parent's argmax,
    so every path must be accepted to its full depth; typical: the oracle's outcome, with the
    usual near-tie allowance."""
    import torch
    from speculative_decoding_heads_amd import api
    choices = seeded_tree_choices(0)
    tree = api.Tree(choices)
    ot = tree_buffers(choices)
    T, B = ot["T"], 3
    say("evaluate_posterior V", V, "offset", off, "mode", mode)
    rng = np.random.default_rng(V + 7 * off + 13 * mode)
    lg, toks = _posterior_case(rng, ot, B, V, mode, match_p=1.0 if mode == GREEDY else 0.7, scale=2.0)
    buf = torch.empty(B * T * V + off, dtype=torch.float32, device=dev)
    buf[off:] = torch.from_numpy(lg.ravel()).to(dev)
    lgd = buf[off:].view(B, T, V)
    assert (lgd.data_ptr() % 16 != 0) == (off % 4 != 0)
    tau, eps, delta = 0.7, 0.09, 0.3
    best, a, sel, nr = api.evaluate_posterior(tree, lgd, torch.from_numpy(toks).to(dev), mode, tau, eps, delta)
    torch.cuda.synchronize()
    got = np.stack([to_np(x) for x in (best, a, sel, nr)], 1)
    if mode == GREEDY:
        assert got[:, 1].tolist() == [ot["D"]] * B
    near = sum(posterior_outcome(ot, lg[b], toks[b], mode, tau, eps, delta, got[b]) for b in range(B))
    assert near <= 1


@pytest.mark.parametrize("dtype_name", ["bf16", "fp32"])
def test_kv_compact_bit_exact(dev, dtype_name):
    import torch
    from speculative_decoding_heads_amd import api
    say("kv_compact", dtype_name)
    tdt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    ot = tree_buffers(PAGE_TREE_CHOICES)
    tree = api.Tree(PAGE_TREE_CHOICES)
    rng = np.random.default_rng(3)
    NL, B, Hkv, Lmax, Dh, T = 3, 4, 2, 50, 64, 64
    Kc = rng.standard_normal((NL, B, Hkv, Lmax, Dh)).astype(np.float32)
    Vc = rng.standard_normal((NL, B, Hkv, Lmax, Dh)).astype(np.float32)
    Kt = rng.standard_normal((NL, B, Hkv, T, Dh)).astype(np.float32)
    Vt = rng.standard_normal((NL, B, Hkv, T, Dh)).astype(np.float32)
    if dtype_name == "bf16":
        from workloads import bf16_round
        Kc, Vc, Kt, Vt = (bf16_round(x) for x in (Kc, Vc, Kt, Vt))
    best = np.array([0, 7, 41, 20], np.int32)
    acc = np.array([4, 3, 0, 2], np.int32)  # within each chosen path's length
    seq = np.array([10, 40, 49, 0], np.int32)
    toks = rng.integers(0, 1000, (B, T)).astype(np.int32)
    d = lambda x: torch.from_numpy(x).to(dev)
    gK, gV = to_dev(Kc, tdt, dev), to_dev(Vc, tdt, dev)
    gseq = d(seq)
    out_tokens = torch.full((B, 16), -1, dtype=torch.int32, device=dev)
    n_out = torch.tensor([0, 3, 16, 1], dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    api.kv_compact(tree, gK, gV, to_dev(Kt, tdt, dev), to_dev(Vt, tdt, dev), d(best), d(acc), gseq, d(toks),
                   out_tokens, n_out, err)
    torch.cuda.synchronize()
    # sequence 2 (seq 49 + 1 > 50 would fit, n_out 16 + 1 > 16 does not) must be untouched and flagged
    rK, rV, rseq = oracle_compact(ot, Kc, Vc, Kt, Vt, best, acc, seq)
    rseq[2] = seq[2]
    rK[:, 2], rV[:, 2] = Kc[:, 2], Vc[:, 2]
    assert np.array_equal(to_np(gK), rK) and np.array_equal(to_np(gV), rV)
    assert to_np(gseq).tolist() == rseq.tolist()
    assert int(to_np(err)[0]) == 1
    ot_ = to_np(out_tokens)
    for b, n0 in [(0, 0), (1, 3), (3, 1)]:
        want = [int(toks[b, ot["retrieve"][best[b], i]]) for i in range(acc[b] + 1)]
        assert ot_[b, n0:n0 + acc[b] + 1].tolist() == want
    assert to_np(n_out).tolist() == [5, 7, 16, 4]


@pytest.mark.parametrize("B", [1, 8])
def test_heads_topk_bf16_full_size(dev, B):
    """Medusa heads at d 4096, V 32000, 4 heads, top-10 (bf16) against the oracle."""
    import torch
    from speculative_decoding_heads_amd import api
    say("medusa_heads_topk bf16 B", B)
    h, W1, W2 = heads_weights(seed=B, B=B)
    tdt = torch.bfloat16
    idx, val = api.medusa_heads_topk(to_dev(h, tdt, dev), to_dev(W1, tdt, dev), to_dev(W2, tdt, dev), 10)
    torch.cuda.synchronize()
    # the ranking is decided on float32 logits on both sides
    ref_logits = medusa_heads_logits(h, W1, W2, bf16=True).astype(np.float32).astype(np.float64)
    check_heads_topk(to_np(idx), to_np(val), ref_logits)


def test_heads_topk_bf16_all_tree_nodes(dev):
    """The heads on every node of 8 sequences' 64-node trees (512 hidden states, the
    square-tile product path), full d / V / H; the oracle checks 6 sampled rows."""
    import torch
    from speculative_decoding_heads_amd import api
    B = 512
    say("medusa_heads_topk bf16 B", B)
    h, W1, W2 = heads_weights(seed=3, B=B)
    tdt = torch.bfloat16
    idx, val = api.medusa_heads_topk(to_dev(h, tdt, dev), to_dev(W1, tdt, dev), to_dev(W2, tdt, dev), 10)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, 400, 511]
    ref_logits = medusa_heads_logits(h[rows], W1, W2, bf16=True).astype(np.float32).astype(np.float64)
    check_heads_topk(to_np(idx)[rows], to_np(val)[rows], ref_logits)


def test_heads_topk_fp32_small(dev):
    import torch
    from speculative_decoding_heads_amd import api
    say("medusa_heads_topk fp32 small")
    rng = np.random.default_rng(0)
    h = rng.standard_normal((3, 64)).astype(np.float32)
    W1 = (rng.standard_normal((2, 64, 64)) * 0.02).astype(np.float32)
    W2 = (rng.standard_normal((2, 512, 64)) * 0.02).astype(np.float32)
    idx, val = api.medusa_heads_topk(*(torch.from_numpy(x).to(dev) for x in (h, W1, W2)), 3)
    torch.cuda.synchronize()
    ref = medusa_heads_logits(h, W1, W2)
    assert np.array_equal(to_np(idx), topk_desc(ref, 3))
    assert_close(to_np(val), np.take_along_axis(ref, topk_desc(ref, 3), -1), rtol=1e-5, atol=1e-6, what="val")


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (8, 1000, 512), (64, 12288, 4096), (64, 4096, 11008),
                                   (100, 384, 256), (512, 512, 4096), (40, 1000, 1056), (33, 200, 96),
                                   # square-tile path (M >= 192, K % 64 == 0): 128-row tiles with ragged M
                                   # and N, a single 64-k chunk, as many chunks as LDS buffers, 256-row
                                   # tiles with ragged M and N; K % 64 != 0 goes to the streaming path
                                   (300, 1000, 512), (256, 512, 64), (512, 4096, 4096), (768, 16484, 256),
                                   (1000, 20000, 128), (192, 256, 32), (700, 300, 96),
                                   # streaming path with three-wave 96-row workgroup tiles (ragged last tile)
                                   (64, 20000, 256),
                                   # streaming path, 128-row workgroup tiles; 48 rows (clamped A rows)
                                   (64, 32000, 256), (48, 5000, 1024),
                                   # few rows with K % 64 != 0: the register-staged 64-row-tile kernel,
                                   # rows past M re-reading the last one
                                   (1, 3000, 1056), (5, 4096, 96), (17, 700, 1056),
                                   # N % 4 != 0: every epilogue's element-by-element stores (direct-load
                                   # tiles; the split-K reduction at M 1; register-staged; square tiles)
                                   (64, 1001, 256), (8, 999, 512), (1, 4095, 4096), (5, 4099, 96),
                                   (300, 1003, 512)])
def test_gemm_bf16(dev, M, N, K):
    import torch
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import EPI_F32
    say("gemm bf16", M, N, K)
    rng = np.random.default_rng(M + N)
    from workloads import bf16_round
    A = bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    W = bf16_round((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    out = api.gemm(to_dev(A, torch.bfloat16, dev), to_dev(W, torch.bfloat16, dev), EPI_F32)
    torch.cuda.synchronize()
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    assert_close(to_np(out), ref, rtol=1e-4, atol=1e-4, what="gemm")


@pytest.mark.parametrize("dtype_name,M", [("bf16", 5), ("fp32", 5), ("bf16", 260)])
def test_gemm_epilogues(dev, dtype_name, M):
    import torch
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import EPI_RESID, EPI_SILU_RESID_A, EPI_STORE, EPI_SWIGLU
    from workloads import bf16_round
    say("gemm epilogues", dtype_name, "M", M)
    tdt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    rnd = bf16_round if dtype_name == "bf16" else (lambda x: x)
    tol = dict(rtol=2e-2, atol=1e-2) if dtype_name == "bf16" else dict(rtol=1e-5, atol=1e-5)
    rng = np.random.default_rng(1)
    K = 256
    A = rnd(rng.standard_normal((M, K)).astype(np.float32))
    W = rnd((rng.standard_normal((512, K)) * 0.05).astype(np.float32))
    R = rnd(rng.standard_normal((M, 512)).astype(np.float32))
    acc = A.astype(np.float64) @ W.astype(np.float64).T
    gA, gW = to_dev(A, tdt, dev), to_dev(W, tdt, dev)
    out = api.gemm(gA, gW, EPI_STORE)
    assert_close(to_np(out), acc, what="store", **tol)
    gR = to_dev(R, tdt, dev)
    out = api.gemm(gA, gW, EPI_RESID, out=gR.clone(), R=gR)
    assert_close(to_np(out), acc + R, what="resid", **tol)
    out = api.gemm(gA, gW, EPI_SWIGLU)
    assert_close(to_np(out), silu(acc[:, 0::2]) * acc[:, 1::2], what="swiglu", **tol)
    Wsq = rnd((rng.standard_normal((2 * K, K)) * 0.05).astype(np.float32))  # two K x K heads stacked
    out = api.gemm(gA, to_dev(Wsq, tdt, dev), EPI_SILU_RESID_A)
    z = A.astype(np.float64) @ Wsq.astype(np.float64).T
    assert_close(to_np(out), np.concatenate([A, A], 1) + silu(z), what="silu_resid", **tol)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M", [5, 64, 260])
def test_gemm_epilogues_odd_widths(dev, M):
    """bf16 store and residual epilogues at N 1001 and SwiGLU at N 514 (257 outputs a
    row): output rows whose stride and width are not multiples of 4 take the
    element-by-element stores; M 260 takes the square-tile kernel."""
    import torch
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import EPI_RESID, EPI_STORE, EPI_SWIGLU
    from workloads import bf16_round
    say("gemm odd-width epilogues M", M)
    tol = dict(rtol=2e-2, atol=1e-2)
    rng = np.random.default_rng(M + 3)
    K = 256
    A = bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    W = bf16_round((rng.standard_normal((1001, K)) * 0.05).astype(np.float32))
    R = bf16_round(rng.standard_normal((M, 1001)).astype(np.float32))
    acc = A.astype(np.float64) @ W.astype(np.float64).T
    gA = to_dev(A, torch.bfloat16, dev)
    gW = to_dev(W, torch.bfloat16, dev)
    out = api.gemm(gA, gW, EPI_STORE)
    assert_close(to_np(out), acc, what="store", **tol)
    gR = to_dev(R, torch.bfloat16, dev)
    out = api.gemm(gA, gW, EPI_RESID, out=gR.clone(), R=gR)
    assert_close(to_np(out), acc + R, what="resid", **tol)
    W2 = bf16_round((rng.standard_normal((514, K)) * 0.05).astype(np.float32))
    acc2 = A.astype(np.float64) @ W2.astype(np.float64).T
    out = api.gemm(gA, to_dev(W2, torch.bfloat16, dev), EPI_SWIGLU)
    assert tuple(out.shape) == (M, 257)
    assert_close(to_np(out), silu(acc2[:, 0::2]) * acc2[:, 1::2], what="swiglu", **tol)
    torch.cuda.synchronize()


def test_gemm_swiglu_96_row_tiles(dev):
    """The gate/up shape of the 7B verify forward (N 22016) takes three-wave 96-row
    workgroup tiles; SwiGLU pairs rows 2j (gate) and 2j+1 (up)."""
    import torch
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import EPI_SWIGLU
    from workloads import bf16_round
    say("gemm swiglu 64 x 22016 x 256")
    rng = np.random.default_rng(7)
    A = bf16_round(rng.standard_normal((64, 256)).astype(np.float32))
    W = bf16_round((rng.standard_normal((22016, 256)) * 0.05).astype(np.float32))
    out = api.gemm(to_dev(A, torch.bfloat16, dev), to_dev(W, torch.bfloat16, dev), EPI_SWIGLU)
    torch.cuda.synchronize()
    acc = A.astype(np.float64) @ W.astype(np.float64).T
    assert_close(to_np(out), silu(acc[:, 0::2]) * acc[:, 1::2], what="swiglu", rtol=2e-2, atol=1e-2)


@pytest.mark.parametrize("dtype_name,M,N,K", [("bf16", 64, 4096, 4096), ("bf16", 64, 4096, 11008),
                                              ("bf16", 5, 512, 256), ("bf16", 40, 1000, 1056),
                                              # K splits of 3 and 5: partial batches of the split loads
                                              ("bf16", 64, 1024, 768), ("bf16", 64, 1024, 1280),
                                              ("fp32", 5, 512, 256)])
def test_gemm_resid_rmsnorm(dev, dtype_name, M, N, K):
    import torch
    from oracle.decoder import rmsnorm
    from speculative_decoding_heads_amd import api
    from workloads import bf16_round
    say("gemm_resid_rmsnorm", dtype_name, M, N, K)
    tdt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    rnd = bf16_round if dtype_name == "bf16" else (lambda x: x)
    tol = dict(rtol=2e-2, atol=1e-2) if dtype_name == "bf16" else dict(rtol=1e-5, atol=1e-5)
    rng = np.random.default_rng(M * 7 + K)
    A = rnd(rng.standard_normal((M, K)).astype(np.float32))
    W = rnd((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    X = rnd(rng.standard_normal((M, N)).astype(np.float32))
    g = rnd((1.0 + 0.1 * rng.standard_normal(N)).astype(np.float32))
    gX = to_dev(X, tdt, dev)
    Y = api.gemm_resid_rmsnorm(to_dev(A, tdt, dev), to_dev(W, tdt, dev), gX, to_dev(g, tdt, dev), 1e-6)
    torch.cuda.synchronize()
    x_ref = X.astype(np.float64) + A.astype(np.float64) @ W.astype(np.float64).T
    assert_close(to_np(gX), x_ref, what="residual", **tol)
    # the norm is taken over the stored residual, so compare it against that
    y_ref = rmsnorm(to_np(gX).astype(np.float64), g)
    assert_close(to_np(Y), y_ref, what="norm", **tol)


def test_argmax_and_topk_rows_ties(dev):
    import torch
    from speculative_decoding_heads_amd import api
    say("argmax/topk rows")
    x = np.zeros((3, 1000), np.float32)
    x[0, [5, 17, 900]] = 2.0
    x[1] = np.random.default_rng(0).standard_normal(1000)
    x[2, 999] = 1.0
    g = torch.from_numpy(x).to(dev)
    am = api.argmax_rows(g)
    idx, val = api.topk_rows(g, 5)
    torch.cuda.synchronize()
    assert to_np(am).tolist() == [5, int(x[1].argmax()), 999]
    assert np.array_equal(to_np(idx), topk_desc(x, 5))


@pytest.mark.parametrize("M,V", [(100, 5000), (2048, 9000), (7, 1001)])
def test_topk_rows_many_rows(dev, M, V):
    """Many rows take longer chunks per wave in the first stage (batched float4 reads
    plus a scalar tail; V % 4 != 0 reads scalars only); ties still go to the lower
    index (values drawn from a small set so that ties are common)."""
    import torch
    from speculative_decoding_heads_amd import api
    say("topk rows M", M, "V", V)
    rng = np.random.default_rng(M)
    x = rng.integers(-50, 50, size=(M, V)).astype(np.float32) / 8.0
    idx, val = api.topk_rows(torch.from_numpy(x).to(dev), 10)
    torch.cuda.synchronize()
    want = topk_desc(x, 10)
    assert np.array_equal(to_np(idx), want)
    assert np.array_equal(to_np(val), np.take_along_axis(x, want, -1))


@pytest.mark.parametrize("V", [1, 3, 17, 64, 65, 100])
def test_topk_and_argmax_short_rows(dev, V):
    """Rows far shorter than a workgroup (most threads hold only padding): random, all
    -inf (the top K are the first K indices), one finite entry among -inf, constant,
    and small integers (many ties); top-K with K = min(V, 10) and the row argmax."""
    import torch
    from speculative_decoding_heads_amd import api
    say("topk / argmax short rows V", V)
    rng = np.random.default_rng(V + 5)
    K = min(V, 10)
    x = np.zeros((5, V), np.float32)
    x[0] = rng.standard_normal(V)
    x[1] = -np.inf
    x[2] = -np.inf
    x[2, V // 2] = -3.0
    x[3] = 0.5
    x[4] = rng.integers(-2, 2, size=V)
    g = torch.from_numpy(x).to(dev)
    idx, val = api.topk_rows(g, K)
    am = api.argmax_rows(g)
    torch.cuda.synchronize()
    want = topk_desc(x, K)
    assert np.array_equal(to_np(idx), want)
    assert np.array_equal(to_np(val), np.take_along_axis(x, want, -1))
    assert to_np(am).tolist() == want[:, 0].tolist()


@pytest.mark.parametrize("V", [2, 5])
@pytest.mark.parametrize("mode", [GREEDY, TYPICAL])
def test_posterior_tiny_vocabulary(dev, V, mode):
    """Vocabularies of 2 and 5 tokens: nearly every thread of the per-node statistics
    holds padding; the outcome equals the oracle's (counted near-ties)."""
    import torch
    from speculative_decoding_heads_amd import api
    say("evaluate_posterior tiny V", V, "mode", mode)
    ot = tree_buffers(PAGE_TREE_CHOICES)
    tree = api.Tree(PAGE_TREE_CHOICES)
    rng = np.random.default_rng(V + 31 * mode)
    B = 4
    lg, toks = _posterior_case(rng, ot, B, V, mode, match_p=0.8, scale=1.5)
    tau, eps, delta = 0.7, 0.09, 0.3
    best, a, sel, nr = api.evaluate_posterior(tree, torch.from_numpy(lg).to(dev), torch.from_numpy(toks).to(dev),
                                              mode, tau, eps, delta)
    torch.cuda.synchronize()
    got = np.stack([to_np(x) for x in (best, a, sel, nr)], 1)
    near = sum(posterior_outcome(ot, lg[b], toks[b], mode, tau, eps, delta, got[b]) for b in range(B))
    assert near <= 1


@pytest.mark.parametrize("V", [8000, 40000])
def test_topk_rows_unaligned_rows(dev, V):
    """Rows whose base is not 16-byte aligned (one float into the buffer) are read as
    scalars: the one-workgroup-per-row kernel (V 8000) and the two-stage path (V 40000);
    values from a small set so that ties are common."""
    import torch
    from speculative_decoding_heads_amd import api
    say("topk rows unaligned V", V)
    rng = np.random.default_rng(V + 1)
    M = 6
    x = rng.integers(-50, 50, size=(M, V)).astype(np.float32) / 8.0
    buf = torch.empty(M * V + 1, dtype=torch.float32, device=dev)
    buf[1:] = torch.from_numpy(x.ravel()).to(dev)
    xd = buf[1:].view(M, V)
    assert xd.data_ptr() % 16 != 0
    idx, val = api.topk_rows(xd, 10)
    torch.cuda.synchronize()
    want = topk_desc(x, 10)
    assert np.array_equal(to_np(idx), want)
    assert np.array_equal(to_np(val), np.take_along_axis(x, want, -1))


# rows of at most 32768 entries take the one-workgroup-per-row kernel, longer ones
# (65537, and 128256 as in a 128k vocabulary) the two-stage path
@pytest.mark.parametrize("V,K", [(32000, 10), (32001, 16), (32768, 1), (4097, 10), (65537, 16), (128256, 10)])
def test_topk_rows_plateaus_and_full_vocab(dev, V, K):
    """Rows of a vocabulary's length: a plain random row, a row of one repeated value
    (every entry ties at the threshold, more than the candidate list holds), a
    plateau with a few larger entries, half-integers, -0 / +0 ties on top of a
    row of -1 (5 of them, and 30 spread out: a short candidate list of ties), and
    100 equal maxima on a random row (a candidate list longer than a wave); the
    exact (value desc, index asc) top K (-0 ties with +0)."""
    import torch
    from speculative_decoding_heads_amd import api
    say("topk rows plateaus V", V, "K", K)
    rng = np.random.default_rng(V + K)
    x = np.zeros((7, V), np.float32)
    x[0] = rng.standard_normal(V)
    x[1] = 0.25
    x[2, rng.choice(V, 5, replace=False)] = 1.0
    x[3] = rng.integers(-3, 3, size=V) / 2.0
    x[4] = -1.0
    x[4, [7, 3, 11, 5, 2]] = [-0.0, 0.0, -0.0, 0.0, -0.0]
    x[5] = -1.0
    x[5, rng.choice(V, 30, replace=False)] = np.where(np.arange(30) % 2 == 0, -0.0, 0.0)
    x[6] = rng.standard_normal(V)
    x[6, rng.choice(V, 100, replace=False)] = 10.0
    idx, val = api.topk_rows(torch.from_numpy(x).to(dev), K)
    torch.cuda.synchronize()
    want = topk_desc(x, K)
    assert np.array_equal(to_np(idx), want)
    assert np.array_equal(to_np(val), np.take_along_axis(x, want, -1))
