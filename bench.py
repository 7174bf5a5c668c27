"""Benchmark: one Medusa tree-verify step of a 7B-shaped random-init decoder on one MI355X.

Workload (the full verify step): 32 layers, d 4096, 32 MHA heads x 128, SwiGLU 11008,
V 32000, 4 Medusa heads, the seeded 64-node tree (top-10, depth <= 4), prefix 1024,
typical acceptance eps 0.09, delta 0.3, temperature 0.7, batch 1, bf16.  A step is one
medusa_step call: heads + top-K, candidate expansion, the verify forward with tree
attention, acceptance, KV compaction, the next root and heads' input.  The prefix is
reset to 1024 tokens before every step (a device-side copy), so every timed step sees
the same workload.

Also measured (same JSON line):
  roofline       the dominant kernel: gemm_dma_kernel on the gate/up projection of the
                 64 tree rows (M 64, N 22016, K 4096, SwiGLU epilogue), the largest
                 single share of the step; average launch time with HIP events over the
                 32 layers' weights, against 8 TB/s; `traffic` from the committed
                 rocprofv3 FETCH_SIZE / WRITE_SIZE summary when the kernel source still
                 matches it.  `step_projections` adds every projection of one step.
  tree_attention the attention kernel alone at batch 8, 32/8 heads, prefix 65536, at
                 batch 1 with the 7B-shaped model's 32 heads (no KV sharing), prefix 65536, and
                 at batch 1, prefix 1024, against 8 TB/s
  prefix_sweep   the same step (eager launches) at prefixes 4k, 16k and 64k, the cache
                 filled with N(0,1) keys and values (5 timed steps each)
  tree_size_sweep
                 the step with trees of 8..64 nodes that medusa_tree_from_acceptance
                 builds from a synthetic per-(depth, rank) acceptance table: step time,
                 the table's expected tokens per step and their ratio
  heads_all_tree_nodes
                 medusa_heads_topk on the hidden states of every node of 8 sequences'
                 64-node trees (512 rows: the heads applied inside the verify forward),
                 against the 2.5 PFLOP/s dense bf16 peak
  tree_attention_sweep
                 the attention kernel alone at prefixes 1k..64k, batch 1 and 8
  heads_topk_candidates
                 heads + top-10 + candidate expansion at batch 1 and 8 (1.18 GB of head
                 weights per call), against 8 TB/s
  kv_compact     the compaction call at batch 8, prefix 65536 (one layer)
  tiny_fp32_step the 2-layer fp32 model's verify step (launch-bound): steps/s, tok/s
  cpu_baseline   the oracle on the host cores on a bounded sample of the same step

python bench.py [--gpus 1] [--steps K] [--warmup W]
python bench.py --roofline-only      the dominant-kernel launches and a 256 MiB copy
                                     (counter calibration) only, for rocprofv3 --pmc
python bench.py --attn-traffic-only  the batch-8 / prefix-65536 attention launches and the
                                     256 MiB copy only, for rocprofv3 --pmc
python bench.py --traffic-from FETCH_DIR WRITE_DIR
                                     turn the two counter runs into the traffic file
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFS = 2500.0  # dense bf16
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_dma_gate_up_M64_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "speculative_decoding_heads_amd", "csrc", "gemm.hip")
COPY_BYTES = 256 << 20  # calibration copy: reads and writes this many bytes


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--prefix", type=int, default=1024)
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--attn-reps", type=int, default=20)
    p.add_argument("--roofline-only", action="store_true")
    p.add_argument("--attn-traffic-only", action="store_true")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    p.add_argument("--sweep", type=str, default="4096,16384,65536",
                   help="longer prefixes at which the same step is also timed ('' for none)")
    return p.parse_args()


class Timer:
    """HIP events on the current torch stream (the stream the library launches on)."""

    def __init__(self):
        import torch
        self.s = torch.cuda.Event(enable_timing=True)
        self.e = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.s.record()
        return self

    def __exit__(self, *a):
        self.e.record()

    def ms(self):
        self.e.synchronize()
        return self.s.elapsed_time(self.e)


def gemm_bytes(M, N, K, out_bytes):
    return N * K * 2 + M * K * 2 + M * N * out_bytes


def gate_up_bytes(M, F, d):
    """Algorithmic bytes of one gate/up launch: W [2F, d] + A [M, d] in, SwiGLU [M, F] out (bf16)."""
    return 2 * F * d * 2 + M * d * 2 + M * F * 2


def source_sha():
    import hashlib
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def read_traffic():
    """HBM bytes per dominant-kernel launch from the committed counter summary, or None
    when the kernel source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_sha():
        return None
    return t.get("bytes_per_launch")


def traffic_from(fetch_dir, write_dir):
    """Average FETCH_SIZE / WRITE_SIZE (KiB) per gate/up launch from two rocprofv3 --pmc
    runs of `bench.py --roofline-only`, each scaled by what the same counter reads for
    the 256 MiB row copy (gather_rows_kernel, which reads and writes COPY_BYTES) in the
    same run, written to the traffic file."""
    import csv
    import glob

    def load(d, counter):
        rows = []
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fn) as f:
                rows += [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        gemm = [float(r["Counter_Value"]) for r in rows if "gemm_dma_kernel" in r["Kernel_Name"]]
        copy = [float(r["Counter_Value"]) for r in rows if "gather_rows_kernel" in r["Kernel_Name"]]
        if not gemm or not copy:
            raise SystemExit("no %s samples for the GEMM or the copy in %s" % (counter, d))
        return float(np.median(gemm)), float(np.median(copy))

    g_f, c_f = load(fetch_dir, "FETCH_SIZE")
    g_w, c_w = load(write_dir, "WRITE_SIZE")
    ref_kib = COPY_BYTES / 1024.0
    sf, sw = ref_kib / c_f, ref_kib / c_w
    fetch_b, write_b = g_f * sf * 1024.0, g_w * sw * 1024.0
    out = {"kernel": "gemm_dma_kernel gate/up M64 N22016 K4096", "source_sha256": source_sha(),
           "fetch_kib_raw": g_f, "write_kib_raw": g_w, "copy_fetch_kib_raw": c_f, "copy_write_kib_raw": c_w,
           "copy_bytes": COPY_BYTES, "fetch_scale": sf, "write_scale": sw,
           "fetch_bytes_per_launch": round(fetch_b), "write_bytes_per_launch": round(write_b),
           "bytes_per_launch": round(fetch_b + write_b),
           "algorithmic_bytes_per_launch": gate_up_bytes(64, 11008, 4096)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import EPI_F32, EPI_RESID, EPI_SWIGLU, TYPICAL, lib
    from speculative_decoding_heads_amd.model import (Model, State, StepGraph, init_topk_carry, prefill, step,
                                                      step_fused, step_fused_workspace_size, step_workspace_size)
    from workloads import (SevenBConfig, acceptance_table, model_weights_torch, prompt_tokens, seeded_tree_choices,
                           torch_normal)

    dev = torch.device("cuda:0")
    cfg = SevenBConfig
    NL = args.layers
    lib()
    if args.attn_traffic_only:
        attn_traffic_run(dev)
        return
    log("generating %d-layer 7B-shaped weights on device" % NL)
    params, heads = model_weights_torch(cfg, 1, dev, torch.bfloat16, n_layers=NL)
    sample_layers = [{k: v for k, v in params["layers"][i].items()} for i in range(min(4, NL))]
    sweep_L = [int(x) for x in args.sweep.split(",") if x.strip()]
    model = Model(params, heads, max_pos=max([args.prefix] + sweep_L) + 512)
    for l in params["layers"]:
        for k in ("wq", "wk", "wv", "w_gate", "w_up"):
            l[k] = None
    torch.cuda.empty_cache()
    tree = api.Tree(seeded_tree_choices(0), K=10)  # the heads' top-10 as the tree's rank stride
    B = 1
    gate_up = make_gate_up(model, cfg, NL, tree.T * B, dev)
    if args.roofline_only:
        from speculative_decoding_heads_amd._lib import check, ptr, stream_ptr
        us = gate_up(2)
        # calibration: a plain row copy of COPY_BYTES (fp32 rows of 8 KiB) through
        # the library's gather_rows kernel (row 0 of each one-row sequence)
        rows = COPY_BYTES // 8192
        src = torch.ones((rows, 1, 2048), dtype=torch.float32, device=dev)
        dst = torch.empty((rows, 2048), dtype=torch.float32, device=dev)
        sel = torch.zeros(rows, dtype=torch.int32, device=dev)
        for _ in range(3):
            check(lib().medusa_gather_rows(0, rows, 1, 2048, ptr(src), ptr(sel), ptr(dst), stream_ptr()))
        torch.cuda.synchronize()
        print(json.dumps({"gate_up_us": round(us, 3), "copy_bytes": COPY_BYTES}), flush=True)
        return
    Lmax = args.prefix + 128
    st = State(model, B, Lmax, 64)
    prompt = prompt_tokens(7, B, args.prefix, cfg.vocab)
    log("prefill of %d tokens" % args.prefix)
    prefill(model, st, torch.from_numpy(prompt.astype(np.int32)).to(dev))
    torch.cuda.synchronize()
    base_seq = st.seq_len.clone()
    base_K = None
    ws = torch.empty(step_workspace_size(model, tree, B, Lmax), dtype=torch.uint8, device=dev)
    acc_sum = torch.zeros(B, dtype=torch.int64, device=dev)
    tau, eps, delta = 0.7, 0.09, 0.3

    def one_step():
        st.seq_len.copy_(base_seq)
        st.n_out.zero_()
        step(model, tree, st, TYPICAL, tau, eps, delta, L_hint=Lmax, ws=ws)

    # eager launches (one library call per step, ~400 kernel launches from the host)
    log("eager: warmup %d steps" % args.warmup)
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with Timer() as te:
        for _ in range(args.steps):
            one_step()
    eager_ms = te.ms() / args.steps
    eager_wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    log("eager step %.3f ms" % eager_ms)

    # the same step captured once into a HIP graph and replayed
    gstream = torch.cuda.Stream()
    graph = StepGraph(model, tree, st, TYPICAL, tau, eps, delta, L_hint=Lmax, ws=ws, stream=gstream)

    def graph_step():
        st.seq_len.copy_(base_seq)
        st.n_out.zero_()
        graph.replay(gstream)

    with torch.cuda.stream(gstream):
        log("graph: warmup %d steps" % args.warmup)
        for _ in range(args.warmup):
            graph_step()
        torch.cuda.synchronize()
        log("timing %d steps" % args.steps)
        acc_sum.zero_()
        t0 = time.perf_counter()
        with Timer() as tm:
            for _ in range(args.steps):
                graph_step()
                acc_sum += st.accept_len
        step_ms = tm.ms() / args.steps
        wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    torch.cuda.synchronize()
    graph_ms = step_ms
    launch = "HIP graph replay of one step (eager launches: %.4f ms/step)" % eager_ms
    if eager_ms < graph_ms:
        # the reported figure is the faster of the two launch modes, both timed above
        step_ms = eager_ms
        wall_ms = eager_wall_ms
        launch = "eager launches, one library call per step (HIP graph replay: %.4f ms/step)" % graph_ms
    assert int(st.err[0]) == 0, "state error flag set"
    mean_tokens = float(acc_sum.sum()) / (args.steps * B) + 1.0
    steps_per_s = 1e3 / step_ms

    # fused draft + verify: the heads on all 64 tree nodes inside the step, the
    # next candidates taken at the selected node (eager launches, same prefix reset)
    fws = torch.empty(step_fused_workspace_size(model, tree, B, Lmax), dtype=torch.uint8, device=dev)
    carry = init_topk_carry(model, tree, st)

    def fused_step():
        st.seq_len.copy_(base_seq)
        st.n_out.zero_()
        step_fused(model, tree, st, carry, TYPICAL, tau, eps, delta, L_hint=Lmax, ws=fws)

    for _ in range(args.warmup):
        fused_step()
    torch.cuda.synchronize()
    with Timer() as tf:
        for _ in range(args.steps):
            fused_step()
    fused_ms = tf.ms() / args.steps
    assert int(st.err[0]) == 0, "state error flag set"
    log("fused draft+verify step %.3f ms" % fused_ms)
    del fws
    log("step %.3f ms (wall %.3f ms), %.1f steps/s, mean tokens/step %.2f" % (step_ms, wall_ms, steps_per_s,
                                                                              mean_tokens))

    # ---- the same step at longer prefixes: the cache holds N(0,1) keys and values
    # (its contents do not change the work), the prefix length is set directly
    sweep = {}
    for Ls in sweep_L:
        st2 = State(model, B, Ls + 128, 64)
        for l in range(NL):
            st2.Kc[l].normal_()
            st2.Vc[l].normal_()
        st2.h_sel.copy_(st.h_sel)
        st2.root.copy_(st.root)
        seq2 = torch.full((B,), Ls, dtype=torch.int32, device=dev)
        ws2 = torch.empty(step_workspace_size(model, tree, B, Ls + 128), dtype=torch.uint8, device=dev)

        def sweep_step():
            st2.seq_len.copy_(seq2)
            st2.n_out.zero_()
            step(model, tree, st2, TYPICAL, tau, eps, delta, L_hint=Ls + 128, ws=ws2)

        for _ in range(2):
            sweep_step()
        torch.cuda.synchronize()
        acc_sum.zero_()
        nrep = 5
        with Timer() as tw:
            for _ in range(nrep):
                sweep_step()
                acc_sum += st2.accept_len
        ms = tw.ms() / nrep
        toks = float(acc_sum.sum()) / (nrep * B) + 1.0
        sweep[str(Ls)] = {"ms_per_step": round(ms, 4), "steps_per_s": round(1e3 / ms, 3),
                          "accepted_tokens_per_step": round(toks, 3), "accepted_tok_per_s": round(1e3 / ms * toks, 2)}
        log("prefix %d: %.3f ms/step, %.1f steps/s" % (Ls, ms, 1e3 / ms))
        del st2, ws2
        torch.cuda.empty_cache()

    # ---- tree size: trees of n nodes built by the library (medusa_tree_from_acceptance)
    # from a synthetic per-(depth, rank) acceptance table; the step time at each size,
    # the table's expected tokens per step, and their ratio (speed vs candidate count)
    calib_acc = acceptance_table(cfg.n_medusa, 10)
    tree_sweep = {}
    for n_nodes in (8, 16, 24, 32, 48, 64):
        t_choices, e_acc = api.tree_from_acceptance(calib_acc, n_nodes)
        tr = api.Tree(t_choices, K=10)
        ws3 = torch.empty(step_workspace_size(model, tr, B, Lmax), dtype=torch.uint8, device=dev)

        def tree_step():
            st.seq_len.copy_(base_seq)
            st.n_out.zero_()
            step(model, tr, st, TYPICAL, tau, eps, delta, L_hint=Lmax, ws=ws3)

        for _ in range(2):
            tree_step()
        torch.cuda.synchronize()
        nrep = 5
        with Timer() as tt:
            for _ in range(nrep):
                tree_step()
        ms = tt.ms() / nrep
        tree_sweep[str(n_nodes)] = {"ms_per_step": round(ms, 4), "expected_tokens_per_step": round(1.0 + e_acc, 4),
                                    "projected_tok_per_s": round((1.0 + e_acc) * 1e3 / ms, 2)}
        log("tree of %d nodes: %.3f ms/step, expected %.3f tokens/step" % (n_nodes, ms, 1.0 + e_acc))
        del tr, ws3
    assert int(st.err[0]) == 0, "state error flag set"

    # ---- dominant kernel: the gate/up projection at M = 64 rows, over the 32 layers' weights
    T = tree.T
    M = B * T
    d, F, V, Hq, Dh = cfg.d, cfg.ffn, cfg.vocab, cfg.n_heads, cfg.head_dim
    gu_us = gate_up(2)
    gu_b = gate_up_bytes(M, F, d)
    gu_gbs = gu_b / (gu_us * 1e-6) / 1e9
    traffic = read_traffic()
    log("gate/up GEMM: %.2f us per launch, %.1f GB/s (traffic %s)" % (gu_us, gu_gbs, traffic))

    # ---- every projection of one step as the verify forward issues them
    from speculative_decoding_heads_amd._lib import check, ptr, stream_ptr
    need = max([lib().medusa_gemm_workspace_size(1, M, n, k, 1) for n, k in [(3 * d, d), (2 * F, d), (V, d)]] +
               [lib().medusa_gemm_resid_rmsnorm_workspace_size(1, M, d, k) for k in (d, F)])
    gws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    xin = torch_normal((M, F), 1.0, 5, dev, torch.bfloat16)
    outf = torch.empty((M, max(3 * d, V)), dtype=torch.float32, device=dev)
    outb = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    resid = torch.zeros((M, d), dtype=torch.bfloat16, device=dev)
    normed = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    gnorm = torch.ones(d, dtype=torch.bfloat16, device=dev)

    def call(A, K, W, N, epi, C, ldc):
        check(lib().medusa_gemm(1, M, N, K, ptr(A), K, 0, ptr(W), 0, ptr(C), ldc, 0, 1, epi, None, 0, 0, ptr(gws),
                                gws.numel(), stream_ptr()))

    def call_rn(A, K, W):
        check(lib().medusa_gemm_resid_rmsnorm(1, M, d, K, ptr(A), K, ptr(W), ptr(resid), ptr(gnorm), 1e-6,
                                              ptr(normed), ptr(gws), gws.numel(), stream_ptr()))

    gemm_launches = []
    for li in range(NL):
        lw = model.keep[li * 6: li * 6 + 6]  # wqkv, wgu, attn_norm, ffn_norm, wo, wd
        wqkv, wgu, wo, wd = lw[0], lw[1], lw[4], lw[5]
        gemm_launches += [
            (lambda w=wqkv: call(xin, d, w, 3 * d, EPI_F32, outf, 3 * d), gemm_bytes(M, 3 * d, d, 4)),
            (lambda w=wo: call_rn(xin, d, w), gemm_bytes(M, d, d, 2) + 2 * M * d * 2),
            (lambda w=wgu: call(xin, d, w, 2 * F, EPI_SWIGLU, outb, F), gate_up_bytes(M, F, d)),
            (lambda w=wd: call_rn(xin, F, w), gemm_bytes(M, d, F, 2) + 2 * M * d * 2),
        ]
    gemm_launches.append((lambda: call(xin, d, model.lm_head, V, EPI_F32, outf, V), gemm_bytes(M, V, d, 4)))
    for f, _ in gemm_launches:
        f()
    torch.cuda.synchronize()
    with Timer() as tg:
        for f, _ in gemm_launches:
            f()
    gemm_ms = tg.ms()
    gemm_b = sum(b for _, b in gemm_launches)
    gemm_gbs = gemm_b / (gemm_ms * 1e-3) / 1e9
    log("projections of one step: %.3f ms, %.1f GB/s" % (gemm_ms, gemm_gbs))

    # ---- tree attention alone
    def attn_case(Bc, L, reps, Hkv=8):
        q = torch_normal((Bc, T, 32, Dh), 1.0, 11, dev, torch.bfloat16)
        # rotate over > 1 GB of distinct K/V at small L so the 256 MB last-level cache cannot serve them
        nbuf = max(1, min(128, int(1.2e9 // (Bc * Hkv * L * Dh * 2 * 2)) + 1))
        Ks = [torch_normal((Bc, Hkv, L, Dh), 1.0, 20 + i, dev, torch.bfloat16) for i in range(nbuf)]
        Vs = [torch_normal((Bc, Hkv, L, Dh), 1.0, 40 + i, dev, torch.bfloat16) for i in range(nbuf)]
        Kt = torch_normal((Bc, Hkv, T, Dh), 1.0, 60, dev, torch.bfloat16)
        Vt = torch_normal((Bc, Hkv, T, Dh), 1.0, 61, dev, torch.bfloat16)
        seq = torch.full((Bc,), L, dtype=torch.int32, device=dev)
        out = torch.empty_like(q)
        aws = torch.empty(max(1, api.tree_attention_workspace_size(1, Bc, T, 32, Hkv, Dh, L)), dtype=torch.uint8,
                          device=dev)
        for i in range(nbuf):
            api.tree_attention(q, Ks[i], Vs[i], seq, Kt, Vt, tree, Dh ** -0.5, out=out, ws=aws)
        torch.cuda.synchronize()
        with Timer() as ta:
            for r in range(reps):
                i = r % nbuf
                api.tree_attention(q, Ks[i], Vs[i], seq, Kt, Vt, tree, Dh ** -0.5, out=out, ws=aws)
        ms = ta.ms() / reps
        nbytes = Bc * Hkv * L * Dh * 2 * 2 + Bc * Hkv * T * Dh * 2 * 2 + 2 * Bc * T * 32 * Dh * 2
        del Ks, Vs
        torch.cuda.empty_cache()
        return ms, nbytes

    a64_ms, a64_b = attn_case(8, 65536, args.attn_reps)
    a1k_ms, a1k_b = attn_case(1, 1024, args.attn_reps * 5)
    # the 7B-shaped model's attention (32 heads, no KV-head sharing) at a long prefix
    amha_ms, amha_b = attn_case(1, 65536, args.attn_reps, Hkv=32)
    amha_gbs = amha_b / (amha_ms * 1e-3) / 1e9
    a64_gbs = a64_b / (a64_ms * 1e-3) / 1e9
    a1k_gbs = a1k_b / (a1k_ms * 1e-3) / 1e9
    log("tree_attention B8 L65536: %.1f us, %.1f GB/s; B1 L1024: %.1f us, %.1f GB/s; 32 MHA heads L65536: %.1f us, "
        "%.1f GB/s" % (a64_ms * 1e3, a64_gbs, a1k_ms * 1e3, a1k_gbs, amha_ms * 1e3, amha_gbs))

    # ---- the Medusa heads on every node of 8 sequences' trees (M = 8 * 64 = 512 hidden
    # states): the heads' products in the compute-bound regime (square-tile kernel)
    Bh = 8 * T
    hh = torch_normal((Bh, cfg.d), 1.0, 77, dev, torch.bfloat16)
    hidx = torch.empty((Bh, cfg.n_medusa, 10), dtype=torch.int32, device=dev)
    hval = torch.empty((Bh, cfg.n_medusa, 10), dtype=torch.float32, device=dev)
    hws = torch.empty(max(1, lib().medusa_heads_topk_workspace_size(1, Bh, cfg.d, cfg.vocab, cfg.n_medusa, 10)),
                      dtype=torch.uint8, device=dev)
    for _ in range(2):
        api.medusa_heads_topk(hh, heads["W1"], heads["W2"], 10, topk_idx=hidx, topk_val=hval, ws=hws)
    torch.cuda.synchronize()
    hreps = 10
    with Timer() as th:
        for _ in range(hreps):
            api.medusa_heads_topk(hh, heads["W1"], heads["W2"], 10, topk_idx=hidx, topk_val=hval, ws=hws)
    heads_ms = th.ms() / hreps
    heads_flop = 2.0 * Bh * cfg.n_medusa * (cfg.d * cfg.d + cfg.vocab * cfg.d)
    heads_tfs = heads_flop / (heads_ms * 1e-3) / 1e12
    log("heads on all tree nodes (M %d): %.1f us, %.1f TFLOP/s" % (Bh, heads_ms * 1e3, heads_tfs))

    # ---- tree attention alone over prefixes 1k..64k at batch 1 and 8 (32/8 heads)
    attn_sweep = {}
    for Bc in (1, 8):
        for Ls in (1024, 2048, 4096, 8192, 16384, 32768, 65536):
            if Bc == 8 and Ls == 65536:
                ms_, b_ = a64_ms, a64_b
            else:
                ms_, b_ = attn_case(Bc, Ls, max(5, args.attn_reps // 2))
            g_ = b_ / (ms_ * 1e-3) / 1e9
            attn_sweep["B%d_L%d" % (Bc, Ls)] = {"us": round(ms_ * 1e3, 2), "achieved": round(g_, 1),
                                                "frac": round(g_ / HBM_PEAK_GBS, 4), "bytes": b_}
    log("tree_attention sweep: " + ", ".join("%s %.1f us" % (k, v["us"]) for k, v in attn_sweep.items()))

    # ---- heads + top-K + candidates at batch 1 and 8 (the heads' 1.18 GB of weights streamed once)
    heads_b = {}
    tree10 = api.Tree(seeded_tree_choices(0), K=10)  # the same tree on a top-10 stride
    W1, W2 = heads["W1"], heads["W2"]
    hbytes = W1.numel() * 2 + W2.numel() * 2
    for Bc in (1, 8):
        hb = torch_normal((Bc, cfg.d), 1.0, 78, dev, torch.bfloat16)
        hidx_b = torch.empty((Bc, cfg.n_medusa, 10), dtype=torch.int32, device=dev)
        hws_b = torch.empty(max(1, lib().medusa_heads_topk_workspace_size(1, Bc, cfg.d, cfg.vocab, cfg.n_medusa, 10)),
                            dtype=torch.uint8, device=dev)
        root_b = torch.zeros(Bc, dtype=torch.int32, device=dev)
        seq_b = torch.full((Bc,), args.prefix, dtype=torch.int32, device=dev)

        def heads_cand():
            api.medusa_heads_topk(hb, W1, W2, 10, topk_idx=hidx_b, ws=hws_b)
            api.tree_build_candidates(tree10, root_b, hidx_b, seq_b)

        for _ in range(2):
            heads_cand()
        torch.cuda.synchronize()
        with Timer() as thb:
            for _ in range(10):
                heads_cand()
        ms_ = thb.ms() / 10
        g_ = hbytes / (ms_ * 1e-3) / 1e9
        heads_b["B%d" % Bc] = {"us": round(ms_ * 1e3, 2), "achieved": round(g_, 1), "unit": "GB/s",
                               "frac": round(g_ / HBM_PEAK_GBS, 4), "bytes": hbytes}
    log("heads + top-K + candidates: " + ", ".join("%s %.1f us" % (k, v["us"]) for k, v in heads_b.items()))

    # ---- KV compaction after acceptance: one layer, batch 8, 8 KV heads, prefix 65536,
    # accepted length a ~ U{0..4} on a seeded leaf path long enough for it
    rng_c = np.random.default_rng(5)
    Bc, Lc = 8, 65536
    Kc5 = torch.zeros((1, Bc, 8, Lc + 128, Dh), dtype=torch.bfloat16, device=dev)
    Vc5 = torch.zeros_like(Kc5)
    Kt5 = torch_normal((1, Bc, 8, T, Dh), 1.0, 90, dev, torch.bfloat16)
    Vt5 = torch_normal((1, Bc, 8, T, Dh), 1.0, 91, dev, torch.bfloat16)
    best_np = rng_c.integers(0, tree.P, Bc)
    acc_np = np.array([rng_c.integers(0, min(5, int(tree.path_len[b_]))) for b_ in best_np])
    best5 = torch.from_numpy(best_np.astype(np.int32)).to(dev)
    acc5 = torch.from_numpy(acc_np.astype(np.int32)).to(dev)
    seq5_0 = torch.full((Bc,), Lc, dtype=torch.int32, device=dev)
    seq5 = seq5_0.clone()
    tt5 = torch.zeros((Bc, T), dtype=torch.int32, device=dev)

    def compact5():
        seq5.copy_(seq5_0)
        api.kv_compact(tree, Kc5, Vc5, Kt5, Vt5, best5, acc5, seq5, tt5)

    for _ in range(3):
        compact5()
    torch.cuda.synchronize()
    with Timer() as tc5:
        for _ in range(20):
            compact5()
    compact_us = tc5.ms() / 20 * 1e3
    compact_bytes = int(2 * 2 * 8 * Dh * 2 * int((acc_np + 1).sum()))
    log("kv_compact B8 L65536 (1 layer): %.1f us per call (with the length reset)" % compact_us)
    del Kc5, Vc5
    torch.cuda.empty_cache()

    # ---- the tiny fp32 step (2-layer decoder, d 64, 2 heads, the 2-head tree): launch-bound
    tiny = tiny_step_rate(dev)
    log("tiny fp32 step: %.1f us, %.0f steps/s" % (tiny["us_per_step"], tiny["steps_per_s"]))

    # ---- oracle on the host cores, bounded sample of the same step
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(params, heads, sample_layers, model, cfg, tree, prompt, args.prefix, dev)

    out = {
        "metric": "tree-verify steps/s (7B-shaped verify step, prefix 1024)",
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, uniform prompt tokens)",
        "config": {"workload": "7B-shaped Medusa verify step: 32 layers, d 4096, 32x128 MHA, SwiGLU 11008, "
                               "V 32000, 4 Medusa heads, seeded 64-node tree, prefix 1024, typical "
                               "eps 0.09 delta 0.3 tau 0.7, batch 1", "layers": NL, "prefix": args.prefix,
                   "batch": B, "tree_nodes": T, "tree_paths": tree.P},
        "accepted_tokens_per_step": round(mean_tokens, 3),
        "accepted_tok_per_s": round(steps_per_s * mean_tokens, 2),
        "wall_ms_per_step": round(wall_ms, 4),
        "launch": launch,
        "roofline": {"kernel": "gemm_dma_kernel<2,3,7>: gate/up projection, M 64, N 22016, K 4096, SwiGLU",
                     "bound": "hbm", "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": gu_b, "us_per_launch": round(gu_us, 3)},
        "step_projections": {"kernels": "gemm_dma_kernel + resid_rmsnorm_kernel: every projection of one step",
                             "achieved": round(gemm_gbs, 1), "unit": "GB/s", "frac": round(gemm_gbs / HBM_PEAK_GBS, 4),
                             "bytes_per_step": gemm_b, "ms_per_step": round(gemm_ms, 4),
                             "calls": len(gemm_launches)},
        "tree_attention": {
            "B8_L65536": {"us": round(a64_ms * 1e3, 2), "achieved": round(a64_gbs, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(a64_gbs / HBM_PEAK_GBS, 4), "bytes": a64_b},
            "B1_L1024": {"us": round(a1k_ms * 1e3, 2), "achieved": round(a1k_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(a1k_gbs / HBM_PEAK_GBS, 4), "bytes": a1k_b},
            "B1_MHA32_L65536": {"us": round(amha_ms * 1e3, 2), "achieved": round(amha_gbs, 1), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(amha_gbs / HBM_PEAK_GBS, 4), "bytes": amha_b}},
        "prefix_sweep": sweep,
        "tree_size_sweep": {"acceptance": "synthetic table: depth d in top-10 with probability 0.75 * 0.85^d, "
                                          "ranks in proportion to 0.5^r (not from the pages)",
                            "trees": "medusa_tree_from_acceptance (n - 1 most probable rank paths)",
                            "sizes": tree_sweep},
        "fused_draft_verify": {"ms_per_step": round(fused_ms, 4), "steps_per_s": round(1e3 / fused_ms, 3),
                               "note": "heads on all 64 tree nodes in the step (M = 64), next candidates at the "
                                       "selected node; the reported step runs the heads on the selected node only"},
        "heads_all_tree_nodes": {
            "kernels": "gemm_tile_kernel (W1 with the SiLU residual, W2 to fp32 logits) + top-K",
            "rows": Bh, "bound": "mfma", "us": round(heads_ms * 1e3, 2), "achieved": round(heads_tfs, 1),
            "peak": MFMA_PEAK_TFS, "unit": "TFLOP/s", "frac": round(heads_tfs / MFMA_PEAK_TFS, 4),
            "flop": heads_flop},
        "tree_attention_sweep": {"heads": "32 query / 8 KV heads x 128, 64-node tree, bf16", "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "cases": attn_sweep},
        "heads_topk_candidates": {"kernels": "medusa_heads_topk (W1, W2 products + top-10) + tree_build_candidates",
                                  "bound": "hbm", "peak": HBM_PEAK_GBS, "cases": heads_b},
        "kv_compact": {"case": "1 layer, batch 8, 8 KV heads x 128, prefix 65536, a ~ U{0..4}",
                       "us_per_call": round(compact_us, 2), "bytes_moved": compact_bytes,
                       "note": "launch-bound: the time includes a 32-byte length reset"},
        "tiny_fp32_step": tiny,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def attn_traffic_run(dev):
    """For rocprofv3 --pmc: three launches of the attention kernel at batch 8, 32/8 heads x 128,
    prefix 65536, the seeded 64-node tree (one K/V set, 2 147 483 648 cache bytes), then three
    256 MiB row copies (gather_rows_kernel) as the counter calibration."""
    import torch
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import check, lib, ptr, stream_ptr
    from workloads import seeded_tree_choices, torch_normal
    tree = api.Tree(seeded_tree_choices(0))
    Bc, Hkv, L, Dh, T = 8, 8, 65536, 128, tree.T
    q = torch_normal((Bc, T, 32, Dh), 1.0, 11, dev, torch.bfloat16)
    Kc = torch_normal((Bc, Hkv, L, Dh), 1.0, 20, dev, torch.bfloat16)
    Vc = torch_normal((Bc, Hkv, L, Dh), 1.0, 40, dev, torch.bfloat16)
    Kt = torch_normal((Bc, Hkv, T, Dh), 1.0, 60, dev, torch.bfloat16)
    Vt = torch_normal((Bc, Hkv, T, Dh), 1.0, 61, dev, torch.bfloat16)
    seq = torch.full((Bc,), L, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    aws = torch.empty(max(1, api.tree_attention_workspace_size(1, Bc, T, 32, Hkv, Dh, L)), dtype=torch.uint8,
                      device=dev)
    for _ in range(3):
        api.tree_attention(q, Kc, Vc, seq, Kt, Vt, tree, Dh ** -0.5, out=out, ws=aws)
    torch.cuda.synchronize()
    rows = COPY_BYTES // 8192
    src = torch.ones((rows, 1, 2048), dtype=torch.float32, device=dev)
    dst = torch.empty((rows, 2048), dtype=torch.float32, device=dev)
    sel = torch.zeros(rows, dtype=torch.int32, device=dev)
    for _ in range(3):
        check(lib().medusa_gather_rows(0, rows, 1, 2048, ptr(src), ptr(sel), ptr(dst), stream_ptr()))
    torch.cuda.synchronize()
    nbytes = Bc * Hkv * L * Dh * 2 * 2 + Bc * Hkv * T * Dh * 2 * 2 + 2 * Bc * T * 32 * Dh * 2
    print(json.dumps({"attn_algorithmic_bytes": nbytes, "copy_bytes": COPY_BYTES}), flush=True)


def tiny_step_rate(dev, steps=16):
    """The tiny fp32 Medusa step (2-layer decoder, d 64, 4 x 16 heads, SwiGLU 128, V 512,
    2 Medusa heads, the 2-head tree, greedy) after a 32-token prefill: microseconds per
    step (HIP events, eager launches) and accepted tokens per step."""
    import torch
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import GREEDY
    from speculative_decoding_heads_amd.model import Model, State, prefill, step, step_workspace_size
    from workloads import TWO_HEAD_CHOICES, TinyConfig, prompt_tokens, tiny_model
    params, heads = tiny_model(0)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    P = dict(params)
    P["embed"], P["final_norm"], P["lm_head"] = up(params["embed"]), up(params["final_norm"]), up(params["lm_head"])
    P["layers"] = [{k: up(v) for k, v in l.items()} for l in params["layers"]]
    model = Model(P, {k: up(v) for k, v in heads.items()}, max_pos=512)
    tree = api.Tree(TWO_HEAD_CHOICES)
    prompt = up(prompt_tokens(100, 1, TinyConfig.prompt_len, TinyConfig.vocab).astype(np.int32))
    st = State(model, 1, 256, 4 * steps)
    ws = torch.empty(max(1, step_workspace_size(model, tree, 1, 256)), dtype=torch.uint8, device=dev)
    prefill(model, st, prompt)
    for _ in range(3):
        step(model, tree, st, GREEDY, L_hint=256, ws=ws)
    torch.cuda.synchronize()
    n0 = int(st.n_out[0])
    with Timer() as t:
        for _ in range(steps):
            step(model, tree, st, GREEDY, L_hint=256, ws=ws)
    us = t.ms() / steps * 1e3
    toks = (int(st.n_out[0]) - n0) / steps
    return {"us_per_step": round(us, 2), "steps_per_s": round(1e6 / us, 1), "accepted_tokens_per_step": round(toks, 3),
            "tok_per_s": round(1e6 / us * toks, 1), "bound": "launch latency"}


def make_gate_up(model, cfg, NL, M, dev):
    """Returns run(rounds): the gate/up projection launched over the NL layers' weights
    `rounds` times after one warm-up round; the average microseconds per launch (HIP
    events on the stream the library launches on)."""
    import torch
    from speculative_decoding_heads_amd._lib import EPI_SWIGLU, check, lib, ptr, stream_ptr
    from workloads import torch_normal
    d, F = cfg.d, cfg.ffn
    A = torch_normal((M, d), 1.0, 5, dev, torch.bfloat16)
    out = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, lib().medusa_gemm_workspace_size(1, M, 2 * F, d, 1)), dtype=torch.uint8, device=dev)
    weights = [model.keep[li * 6 + 1] for li in range(NL)]

    def launch(w):
        check(lib().medusa_gemm(1, M, 2 * F, d, ptr(A), d, 0, ptr(w), 0, ptr(out), F, 0, 1, EPI_SWIGLU, None, 0, 0,
                                ptr(ws), ws.numel(), stream_ptr()))

    def run(rounds):
        for w in weights:
            launch(w)
        torch.cuda.synchronize()
        with Timer() as t:
            for _ in range(rounds):
                for w in weights:
                    launch(w)
        return t.ms() * 1e3 / (rounds * len(weights))

    return run


def cpu_baseline(params, heads, sample_layers, model, cfg, tree, prompt, prefix, dev):
    """Oracle (NumPy float64) on a bounded sample of one verify step, scaled to steps/s.

    Sample: the Medusa heads on one hidden state, two of the 32 decoder layers over the
    64 tree tokens with a 1024-token prefix, the LM head, and the acceptance rule.  The
    per-step time is heads + 16 x (two layers) + LM head + acceptance."""
    import torch
    from oracle.decoder import forward as oracle_forward
    from oracle.heads import medusa_heads_topk
    from oracle.posterior import TYPICAL, evaluate_posterior_one
    from oracle.tree import tree_buffers
    from workloads import seeded_tree_choices
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    log("cpu baseline: copying a sample of the weights to the host")
    f32 = lambda t: t.float().cpu().numpy()
    nl = len(sample_layers)
    p = dict(n_heads=cfg.n_heads, n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, norm_eps=cfg.norm_eps,
             rope_theta=cfg.rope_theta, embed=f32(model.embed), final_norm=f32(model.final_norm),
             lm_head=f32(model.lm_head),
             layers=[{k: f32(v) for k, v in l.items()} for l in sample_layers])
    W1, W2 = f32(model.W1), f32(model.W2)
    ot = tree_buffers(seeded_tree_choices(0))
    rng = np.random.default_rng(0)
    T = ot["T"]
    Hkv, Dh = cfg.n_kv_heads, cfg.head_dim
    Kc = rng.standard_normal((nl, 1, Hkv, prefix, Dh)).astype(np.float32)
    Vc = rng.standard_normal((nl, 1, Hkv, prefix, Dh)).astype(np.float32)
    toks = rng.integers(0, cfg.vocab, (1, T))
    pos = prefix + ot["depth"][None, :]
    h = rng.standard_normal((1, cfg.d)).astype(np.float32)
    log("cpu baseline: timing the oracle")
    per_steps, total = [], 0.0
    for rep in range(3):
        t0 = time.perf_counter()
        medusa_heads_topk(h, W1, W2, 10, bf16=True)
        t_heads = time.perf_counter() - t0
        t0 = time.perf_counter()
        lg, hh, _, _ = oracle_forward(p, toks, pos, Kc, Vc, np.array([prefix]), ot["anc"], bf16=True, layers=nl)
        t_fwd = time.perf_counter() - t0  # includes the LM head once
        t0 = time.perf_counter()
        evaluate_posterior_one(ot, lg[0], toks[0], TYPICAL, 0.7, 0.09, 0.3)
        t_post = time.perf_counter() - t0
        t0 = time.perf_counter()
        _ = hh[0] @ p["lm_head"].astype(np.float64).T
        t_lm = time.perf_counter() - t0
        per_steps.append(t_heads + (t_fwd - t_lm) * (cfg.n_layers / nl) + t_lm + t_post)
        total += t_heads + t_fwd + t_post + t_lm
        log("cpu baseline rep %d: %.2f s per step" % (rep, per_steps[-1]))
    per_step = float(np.median(per_steps))
    log("cpu baseline: %.1f s of oracle work, median %.2f s per step" % (total, per_step))
    return {"value": round(1.0 / per_step, 5), "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": "heads on one hidden state + %d of %d decoder layers over the 64 tree tokens at prefix "
                      "%d + LM head + typical acceptance, float64 NumPy; per-step time scaled by %d/%d for "
                      "the layers; median of 3 repetitions (%.1f s measured)" % (nl, cfg.n_layers, prefix,
                                                                                  cfg.n_layers, nl, total)}


if __name__ == "__main__":
    main()
