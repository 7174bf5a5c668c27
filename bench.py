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
  sampled_step   the same 7B step with sampled (non-fast) acceptance: a typical draw at
                 every tree node, the next root drawn at the selected node
  read_ceiling   the library's streaming-read kernel over 4 GiB: the practical HBM read
                 rate; every memory-bound entry also reports frac_of_achievable against it
  cpu_baseline   the oracle on the host cores on a bounded sample of the same step, plus
                 the oracle's time on each of the other workloads (oracle_by_config)

Short kernels (attention at small prefixes, KV compaction, the tiny step) are timed as
many back-to-back launches captured in one HIP graph, so the figures are kernel times,
not host launch rates.

python bench.py [--gpus 1] [--steps K] [--warmup W]
python bench.py --roofline-only      the dominant-kernel launches and a 256 MiB copy
                                     (counter calibration) only, for rocprofv3 --pmc
python bench.py --attn-traffic-only  the batch-8 / prefix-65536 attention launches and the
                                     256 MiB copy only, for rocprofv3 --pmc
python bench.py --traffic-from FETCH_DIR WRITE_DIR
                                     turn the two counter runs into the traffic file
python bench.py --heads-only         the heads on 512 tree-node rows (the square-tile
                                     product) only, for rocprofv3 --pmc
python bench.py --summarize-trace DIR
                                     per-kernel, per-launch-shape table (markdown) of a
                                     rocprofv3 --kernel-trace output directory
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
    p.add_argument("--roofline-only", action="store_true",
                   help="for rocprofv3 --pmc: the gate/up projection over the 32 layers' weights, a 256 MiB row copy "
                        "and 1 GiB streaming reads at 256 and 2048 workgroups")
    p.add_argument("--attn-traffic-only", action="store_true")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    p.add_argument("--heads-only", action="store_true")
    p.add_argument("--attn-case", metavar="B,L[,HKV]",
                   help="time one tree-attention case alone (32 query heads x 128, the seeded 64-node tree) as "
                        "back-to-back launches in one HIP graph, for a kernel trace of that case")
    p.add_argument("--summarize-trace", metavar="DIR")
    p.add_argument("--trace-window", metavar="KERNEL:N",
                   help="with --summarize-trace: only the kernels between the N-th and (N+1)-th launch of KERNEL")
    p.add_argument("--trace-runs", metavar="KERNEL",
                   help="with --summarize-trace: consecutive runs of KERNEL launches with one grid, in trace order")
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


def graph_time_us(calls, reps=5):
    """Microseconds per call of `calls` (a list of no-argument launch functions that
    allocate nothing), all captured back to back into one HIP graph and replayed `reps`
    times after one warm-up replay, timed with HIP events on the replaying stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        for f in calls:
            f()
    g.replay()
    torch.cuda.synchronize()
    with Timer() as t:
        for _ in range(reps):
            g.replay()
    us = t.ms() * 1e3 / (reps * len(calls))
    del g
    return us


def read_ceiling(dev, nbytes=4 << 30, reps=10):
    """The library's streaming-read kernel over nbytes (> the 256 MB last-level cache):
    GB/s of 10 back-to-back passes, 2048 workgroups (8 per CU)."""
    import torch
    from speculative_decoding_heads_amd._lib import check, lib, ptr, stream_ptr
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(2048, dtype=torch.int32, device=dev)

    def one():
        check(lib().medusa_read_probe(ptr(buf), nbytes, 2048, ptr(sink), stream_ptr()))

    for _ in range(2):
        one()
    torch.cuda.synchronize()
    with Timer() as t:
        for _ in range(reps):
            one()
    ms = t.ms() / reps
    del buf
    torch.cuda.empty_cache()
    return {"kernel": "read_probe_kernel (16-byte loads, 2048 workgroups)", "bytes": nbytes,
            "us": round(ms * 1e3, 2), "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def _short_kernel_name(name):
    for junk in ("void ", "medusa::", "(anonymous namespace)::", "at::native::"):
        name = name.replace(junk, "")
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):  # drop the parameter list
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            cut = i
            break
    return name[:cut][:80]


def summarize_trace(d, window=None, runs=None):
    """Markdown tables of a rocprofv3 kernel trace: per kernel and launch shape (grid in
    work-items), calls, average / min / max microseconds and share of the kernel time;
    `window` = (kernel, n) restricts it to the dispatches between the n-th and (n+1)-th
    launch of that kernel (one step) and adds the window's wall time; `runs` = kernel
    lists the consecutive runs of that kernel's launches with one grid, in trace order."""
    import csv
    import glob
    rows = []
    for fn in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit("no kernel_trace.csv under %s" % d)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        r["name"] = _short_kernel_name(r["Kernel_Name"])
        r["grid"] = "%s x %s x %s" % (r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"])
        r["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out = []
    if runs:
        out += ["| Run | `%s` grid (work-items) | Launches | Avg (us) | Min (us) | Max (us) |" % runs,
                "|---:|---|---:|---:|---:|---:|"]
        seq, cur = [], None
        for r in rows:
            if runs not in r["name"]:
                continue
            if cur is None or cur[0] != r["grid"]:
                cur = (r["grid"], [])
                seq.append(cur)
            cur[1].append(r["us"])
        for i, (grid, v) in enumerate(seq):
            out.append("| %d | %s | %d | %.2f | %.2f | %.2f |" % (i, grid, len(v), sum(v) / len(v), min(v), max(v)))
        print("\n".join(out))
        return
    if window:
        kname, n = window.rsplit(":", 1)
        idx = [i for i, r in enumerate(rows) if kname in r["name"]]
        n = int(n)
        if n + 1 >= len(idx):
            raise SystemExit("fewer than %d launches of %s" % (n + 2, kname))
        rows = rows[idx[n]:idx[n + 1]]
        wall = (int(rows[-1]["End_Timestamp"]) - int(rows[0]["Start_Timestamp"])) / 1e3
        out.append("Window: launches %d..%d of the trace, between launches %d and %d of `%s`; wall %.1f us, kernel "
                   "time %.1f us.\n" % (idx[n], idx[n + 1] - 1, n, n + 1, kname, wall, sum(r["us"] for r in rows)))
    groups = {}
    for r in rows:
        groups.setdefault((r["name"], r["grid"]), []).append(r["us"])
    total = sum(sum(v) for v in groups.values())
    out += ["| Kernel | Grid (work-items) | Calls | Avg (us) | Min (us) | Max (us) | Total (us) | % of kernel time |",
            "|---|---|---:|---:|---:|---:|---:|---:|"]
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append("| `%s` | %s | %d | %.2f | %.2f | %.2f | %.1f | %.1f |" % (
            name.replace("|", "/"), grid, len(v), sum(v) / len(v), min(v), max(v), sum(v), 100 * sum(v) / total))
    print("\n".join(out))


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
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.trace_window, args.trace_runs)
        return
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import EPI_F32, EPI_RESID, EPI_SWIGLU, SAMPLE_TYPICAL, SAMPLED, TYPICAL, lib
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
    if args.heads_only:
        heads_only_run(dev)
        return
    if args.attn_case:
        attn_case_run(dev, *[int(x) for x in args.attn_case.split(",")])
        return
    log("generating %d-layer 7B-shaped weights on device" % NL)
    params, heads = model_weights_torch(cfg, 1, dev, torch.bfloat16, n_layers=NL)
    sample_layers = [{k: v for k, v in params["layers"][i].items()} for i in range(min(8, NL))]
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
        del src, dst
        # plain streaming reads of 1 GiB beside it (for latency counters): one
        # workgroup per CU, then eight
        rp = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
        sink = torch.empty(2048, dtype=torch.int32, device=dev)
        for nwg in (256, 2048):
            for _ in range(3):
                check(lib().medusa_read_probe(ptr(rp), rp.numel() * 4, nwg, ptr(sink), stream_ptr()))
        torch.cuda.synchronize()
        print(json.dumps({"gate_up_us": round(us, 3), "copy_bytes": COPY_BYTES}), flush=True)
        return
    Lmax = args.prefix + 128
    # output room for every step of a timed block (a step appends at most the tree
    # depth + 1 <= 5 tokens): the output count then only needs a reset per block
    max_new = 6 * max(args.steps, args.warmup, 10)
    st = State(model, B, Lmax, max_new)
    prompt = prompt_tokens(7, B, args.prefix, cfg.vocab)
    log("prefill of %d tokens" % args.prefix)
    prefill(model, st, torch.from_numpy(prompt.astype(np.int32)).to(dev))
    torch.cuda.synchronize()
    base_seq = st.seq_len.clone()
    base_K = None
    ws = torch.empty(step_workspace_size(model, tree, B, Lmax), dtype=torch.uint8, device=dev)
    tau, eps, delta = 0.7, 0.09, 0.3

    # Each step starts from the same 1024-token prefix (the sequence length is
    # reset, one small copy); the appended tokens accumulate in the state's output
    # count over a block, which gives the mean tokens per step afterwards.
    def one_step():
        st.seq_len.copy_(base_seq)
        step(model, tree, st, TYPICAL, tau, eps, delta, L_hint=Lmax, ws=ws)

    # eager launches (one library call per step, ~270 kernel launches from the host)
    log("eager: warmup %d steps" % args.warmup)
    st.n_out.zero_()
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    st.n_out.zero_()
    t0 = time.perf_counter()
    with Timer() as te:
        for _ in range(args.steps):
            one_step()
    eager_ms = te.ms() / args.steps
    eager_wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    log("eager step %.3f ms" % eager_ms)
    mean_tokens = float(st.n_out.sum()) / (args.steps * B)

    # the same step captured once into a HIP graph and replayed
    gstream = torch.cuda.Stream()
    graph = StepGraph(model, tree, st, TYPICAL, tau, eps, delta, L_hint=Lmax, ws=ws, stream=gstream)

    def graph_step():
        st.seq_len.copy_(base_seq)
        graph.replay(gstream)

    with torch.cuda.stream(gstream):
        log("graph: warmup %d steps" % args.warmup)
        st.n_out.zero_()
        for _ in range(args.warmup):
            graph_step()
        st.n_out.zero_()
        torch.cuda.synchronize()
        log("timing %d steps" % args.steps)
        t0 = time.perf_counter()
        with Timer() as tm:
            for _ in range(args.steps):
                graph_step()
        graph_ms = tm.ms() / args.steps
        graph_wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    torch.cuda.synchronize()
    # order check: short alternating blocks of both modes after the main windows
    alt = {"eager": [], "graph": []}
    for _ in range(2):
        st.n_out.zero_()
        with Timer() as ta:
            for _ in range(5):
                one_step()
        alt["eager"].append(round(ta.ms() / 5, 4))
        with torch.cuda.stream(gstream):
            st.n_out.zero_()
            with Timer() as tb:
                for _ in range(5):
                    graph_step()
            alt["graph"].append(round(tb.ms() / 5, 4))
        torch.cuda.synchronize()
    if eager_ms <= graph_ms:
        # the reported figure is the faster of the two launch modes, both timed over the K steps
        step_ms, wall_ms = eager_ms, eager_wall_ms
        launch = "eager launches, one library call per step (HIP graph replay: %.4f ms/step)" % graph_ms
    else:
        step_ms, wall_ms = graph_ms, graph_wall_ms
        launch = "HIP graph replay of one step (eager launches: %.4f ms/step)" % eager_ms
    launch_detail = {"eager_ms": round(eager_ms, 4), "graph_ms": round(graph_ms, 4),
                     "alternating_5_step_blocks_ms": alt}
    assert int(st.err[0]) == 0, "state error flag set"
    steps_per_s = 1e3 / step_ms

    # sampled (non-fast) acceptance: a typical draw at every tree node, the next root
    # drawn at the selected node (eager launches, the same prefix reset)
    samp = dict(kind=SAMPLE_TYPICAL, temperature=tau, eps=eps, delta=delta, top_p=0.8, seed=1234)
    sst = State(model, B, Lmax, max_new, sampling=samp)
    for name in ("Kc", "Vc", "root", "h_sel"):
        getattr(sst, name).copy_(getattr(st, name))

    def sampled_step():
        sst.seq_len.copy_(base_seq)
        step(model, tree, sst, SAMPLED, L_hint=Lmax, ws=ws)

    sst.n_out.zero_()
    for _ in range(args.warmup):
        sampled_step()
    torch.cuda.synchronize()
    sst.n_out.zero_()
    with Timer() as tsm:
        for _ in range(args.steps):
            sampled_step()
    sampled_ms = tsm.ms() / args.steps
    sampled_tokens = float(sst.n_out.sum()) / (args.steps * B)
    assert int(sst.err[0]) == 0, "state error flag set"
    log("sampled step %.3f ms" % sampled_ms)
    del sst

    # fused draft + verify: the heads on all 64 tree nodes inside the step, the
    # next candidates taken at the selected node (eager launches, same prefix reset)
    fws = torch.empty(step_fused_workspace_size(model, tree, B, Lmax), dtype=torch.uint8, device=dev)
    carry = init_topk_carry(model, tree, st)

    def fused_step():
        st.seq_len.copy_(base_seq)
        step_fused(model, tree, st, carry, TYPICAL, tau, eps, delta, L_hint=Lmax, ws=fws)

    st.n_out.zero_()
    for _ in range(args.warmup):
        fused_step()
    torch.cuda.synchronize()
    st.n_out.zero_()
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
        st2 = State(model, B, Ls + 128, 64)  # 5 timed steps after 2 untimed, the output count reset between
        for l in range(NL):
            st2.Kc[l].normal_()
            st2.Vc[l].normal_()
        st2.h_sel.copy_(st.h_sel)
        st2.root.copy_(st.root)
        seq2 = torch.full((B,), Ls, dtype=torch.int32, device=dev)
        ws2 = torch.empty(step_workspace_size(model, tree, B, Ls + 128), dtype=torch.uint8, device=dev)

        def sweep_step():
            st2.seq_len.copy_(seq2)
            step(model, tree, st2, TYPICAL, tau, eps, delta, L_hint=Ls + 128, ws=ws2)

        for _ in range(2):
            sweep_step()
        torch.cuda.synchronize()
        st2.n_out.zero_()
        nrep = 5
        with Timer() as tw:
            for _ in range(nrep):
                sweep_step()
        ms = tw.ms() / nrep
        toks = float(st2.n_out.sum()) / (nrep * B)
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
            step(model, tr, st, TYPICAL, tau, eps, delta, L_hint=Lmax, ws=ws3)

        st.n_out.zero_()
        for _ in range(2):
            tree_step()
        torch.cuda.synchronize()
        st.n_out.zero_()
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
        return attn_case_time(dev, tree, Bc, L, reps, Hkv)

    a64_ms, a64_b = attn_case(8, 65536, args.attn_reps)
    a1k_ms, a1k_b = attn_case(1, 1024, 128)
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
            elif Bc == 1 and Ls == 1024:
                ms_, b_ = a1k_ms, a1k_b
            else:
                ms_, b_ = attn_case(Bc, Ls, max(10, min(128, int(2e6 // Ls))))
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
    n_comp = 100

    def compact_case(NLc, Bc, Hkvc, Lc):
        """n_comp back-to-back compaction calls in one captured graph (each call appends its
        rows after the previous call's, so the cache has room for all of them)."""
        Kc5 = torch.zeros((NLc, Bc, Hkvc, Lc + 6 * n_comp + 8, Dh), dtype=torch.bfloat16, device=dev)
        Vc5 = torch.zeros_like(Kc5)
        Kt5 = torch_normal((NLc, Bc, Hkvc, T, Dh), 1.0, 90, dev, torch.bfloat16)
        Vt5 = torch_normal((NLc, Bc, Hkvc, T, Dh), 1.0, 91, dev, torch.bfloat16)
        best_np = rng_c.integers(0, tree.P, Bc)
        acc_np = np.array([rng_c.integers(0, min(5, int(tree.path_len[b_]))) for b_ in best_np])
        best5 = torch.from_numpy(best_np.astype(np.int32)).to(dev)
        acc5 = torch.from_numpy(acc_np.astype(np.int32)).to(dev)
        seq5 = torch.full((Bc,), Lc, dtype=torch.int32, device=dev)
        tt5 = torch.zeros((Bc, T), dtype=torch.int32, device=dev)
        calls = [lambda: api.kv_compact(tree, Kc5, Vc5, Kt5, Vt5, best5, acc5, seq5, tt5)] * n_comp
        us = graph_time_us(calls, reps=1)
        moved = int(NLc * Hkvc * Dh * 2 * 2 * 2 * int((acc_np + 1).sum()))  # K and V rows, read + write
        del Kc5, Vc5
        torch.cuda.empty_cache()
        return {"us_per_call": round(us, 2), "bytes_moved": moved, "achieved": round(moved / (us * 1e-6) / 1e9, 1),
                "unit": "GB/s", "accepted_rows": (acc_np + 1).tolist()}

    compact5 = compact_case(1, 8, 8, 65536)
    compact5["case"] = "1 layer, batch 8, 8 KV heads x 128, prefix 65536, a ~ U{0..4} on seeded leaves"
    compact_step = compact_case(NL, 1, cfg.n_kv_heads, args.prefix)
    compact_step["case"] = "%d layers, batch 1, 32 KV heads x 128, prefix %d (the verify step's compaction)" % (
        NL, args.prefix)
    log("kv_compact: %.2f us (batch 8, 1 layer), %.2f us (the step's %d layers)" % (
        compact5["us_per_call"], compact_step["us_per_call"], NL))

    # ---- the tiny fp32 step (2-layer decoder, d 64, 2 heads, the 2-head tree): launch-bound
    tiny = tiny_step_rate(dev)
    log("tiny fp32 step: %.1f us, %.0f steps/s" % (tiny["us_per_step"], tiny["steps_per_s"]))

    # ---- the practical HBM read rate: every memory-bound figure also against it
    ceil = read_ceiling(dev)
    ach = ceil["achieved"]
    log("streaming read ceiling: %.1f GB/s" % ach)
    foa = lambda gbs: round(gbs / ach, 4)
    for case in attn_sweep.values():
        case["frac_of_achievable"] = foa(case["achieved"])
    for case in heads_b.values():
        case["frac_of_achievable"] = foa(case["achieved"])
    # the whole step's algorithmic bytes: every projection's weights, activations and
    # outputs, the heads' weights, and per layer the attention's cache, tree K/V, q and out
    attn_layer_b = B * cfg.n_kv_heads * (args.prefix * Dh * 2 * 2 + T * Dh * 2 * 2) + 2 * B * T * Hq * Dh * 2
    step_b = gemm_b + hbytes + NL * attn_layer_b
    step_gbs = step_b / (step_ms * 1e-3) / 1e9

    # ---- oracle on the host cores, bounded sample of the same step
    cpu = None
    if not args.no_cpu_baseline:
        gpu_ref = {"tiny_us": tiny["us_per_step"], "attn_b1_us": round(a1k_ms * 1e3, 2),
                   "heads_b1_us": heads_b["B1"]["us"], "attn_b8_us": round(a64_ms * 1e3, 2),
                   "compact_us": compact5["us_per_call"]}
        cpu = cpu_baseline(params, heads, sample_layers, model, cfg, tree, prompt, args.prefix, dev, gpu_ref)

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
        "launch_detail": launch_detail,
        "roofline": {"kernel": "gemm_dma_kernel<2,3,4>: gate/up projection, M 64, N 22016, K 4096, SwiGLU",
                     "bound": "hbm", "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "achievable": ach, "frac_of_achievable": foa(gu_gbs),
                     "bytes_per_launch": gu_b, "us_per_launch": round(gu_us, 3)},
        "step_hbm": {"bytes_per_step": step_b, "achieved": round(step_gbs, 1), "unit": "GB/s",
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4), "frac_of_achievable": foa(step_gbs),
                     "note": "algorithmic bytes of the whole step (projection and head weights, activations, "
                             "attention cache and tree K/V) over the reported step time"},
        "read_ceiling": ceil,
        "step_projections": {"kernels": "gemm_dma_kernel + resid_rmsnorm_kernel: every projection of one step",
                             "achieved": round(gemm_gbs, 1), "unit": "GB/s", "frac": round(gemm_gbs / HBM_PEAK_GBS, 4),
                             "frac_of_achievable": foa(gemm_gbs), "bytes_per_step": gemm_b,
                             "ms_per_step": round(gemm_ms, 4), "calls": len(gemm_launches)},
        "tree_attention": {
            "B8_L65536": {"us": round(a64_ms * 1e3, 2), "achieved": round(a64_gbs, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(a64_gbs / HBM_PEAK_GBS, 4),
                          "frac_of_achievable": foa(a64_gbs), "bytes": a64_b},
            "B1_L1024": {"us": round(a1k_ms * 1e3, 2), "achieved": round(a1k_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(a1k_gbs / HBM_PEAK_GBS, 4),
                         "frac_of_achievable": foa(a1k_gbs), "bytes": a1k_b},
            "B1_MHA32_L65536": {"us": round(amha_ms * 1e3, 2), "achieved": round(amha_gbs, 1), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(amha_gbs / HBM_PEAK_GBS, 4),
                                "frac_of_achievable": foa(amha_gbs), "bytes": amha_b},
            "timing": "launches captured back to back in one HIP graph, K/V rotated over > 1 GB at short prefixes"},
        "sampled_step": {"ms_per_step": round(sampled_ms, 4), "steps_per_s": round(1e3 / sampled_ms, 3),
                         "accepted_tokens_per_step": round(sampled_tokens, 3),
                         "sampling": "typical draws (tau 0.7, eps 0.09, delta 0.3, Philox seed 1234) at every tree "
                                     "node, candidates accepted when equal to the draw at their parent, eager launches"},
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
        "kv_compact": {"kernels": "compact_kv_kernel + compact_finalize_kernel, %d calls captured in one graph"
                                  % n_comp, "bound": "latency (a few hundred KB per call)",
                       "B8_L65536_1layer": compact5, "step_32layers": compact_step},
        "tiny_fp32_step": tiny,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def attn_case_time(dev, tree, Bc, L, reps, Hkv=8, Dh=128):
    """(ms per call, algorithmic bytes) of tree_attention at batch Bc, prefix L, 32 query /
    Hkv KV heads x Dh: `reps` (at least one full rotation of the K/V sets) launches captured
    in one HIP graph; at short prefixes the launches rotate over > 1 GB of distinct K/V so
    the 256 MB last-level cache cannot serve them."""
    import torch
    from speculative_decoding_heads_amd import api
    from workloads import torch_normal
    T = tree.T
    q = torch_normal((Bc, T, 32, Dh), 1.0, 11, dev, torch.bfloat16)
    nbuf = max(1, min(128, int(1.2e9 // (Bc * Hkv * L * Dh * 2 * 2)) + 1))
    Ks = [torch_normal((Bc, Hkv, L, Dh), 1.0, 20 + i, dev, torch.bfloat16) for i in range(nbuf)]
    Vs = [torch_normal((Bc, Hkv, L, Dh), 1.0, 40 + i, dev, torch.bfloat16) for i in range(nbuf)]
    Kt = torch_normal((Bc, Hkv, T, Dh), 1.0, 60, dev, torch.bfloat16)
    Vt = torch_normal((Bc, Hkv, T, Dh), 1.0, 61, dev, torch.bfloat16)
    seq = torch.full((Bc,), L, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    aws = torch.empty(max(1, api.tree_attention_workspace_size(1, Bc, T, 32, Hkv, Dh, L)), dtype=torch.uint8,
                      device=dev)
    n = max(reps, nbuf)
    calls = [lambda i=i: api.tree_attention(q, Ks[i % nbuf], Vs[i % nbuf], seq, Kt, Vt, tree, Dh ** -0.5, out=out,
                                            ws=aws) for i in range(n)]
    ms = graph_time_us(calls, reps=3) * 1e-3
    nbytes = Bc * Hkv * L * Dh * 2 * 2 + Bc * Hkv * T * Dh * 2 * 2 + 2 * Bc * T * 32 * Dh * 2
    del Ks, Vs
    torch.cuda.empty_cache()
    return ms, nbytes


def attn_case_run(dev, Bc, L, Hkv=8):
    """One attention case alone (for a per-case kernel trace): its time per call and GB/s."""
    from speculative_decoding_heads_amd import api
    from workloads import seeded_tree_choices
    tree = api.Tree(seeded_tree_choices(0))
    ms, nbytes = attn_case_time(dev, tree, Bc, L, max(10, min(128, int(2e6 // L))), Hkv)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"case": "B%d_L%d_Hkv%d" % (Bc, L, Hkv), "us": round(ms * 1e3, 2), "bytes": nbytes,
                      "achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}), flush=True)


def heads_only_run(dev):
    """For rocprofv3 --pmc: the Medusa heads (d 4096, V 32000, 4 heads, top-10) on 512 hidden
    states -- every node of 8 sequences' 64-node trees, the square-tile products -- three times."""
    import torch
    from speculative_decoding_heads_amd import api
    from speculative_decoding_heads_amd._lib import lib
    from workloads import SevenBConfig, torch_normal
    cfg = SevenBConfig
    W1 = torch_normal((cfg.n_medusa, cfg.d, cfg.d), 0.02, 3001, dev, torch.bfloat16)
    W2 = torch_normal((cfg.n_medusa, cfg.vocab, cfg.d), 0.02, 3002, dev, torch.bfloat16)
    hh = torch_normal((512, cfg.d), 1.0, 77, dev, torch.bfloat16)
    idx = torch.empty((512, cfg.n_medusa, 10), dtype=torch.int32, device=dev)
    val = torch.empty((512, cfg.n_medusa, 10), dtype=torch.float32, device=dev)
    ws = torch.empty(lib().medusa_heads_topk_workspace_size(1, 512, cfg.d, cfg.vocab, cfg.n_medusa, 10),
                     dtype=torch.uint8, device=dev)
    for _ in range(3):
        api.medusa_heads_topk(hh, W1, W2, 10, topk_idx=idx, topk_val=val, ws=ws)
    torch.cuda.synchronize()
    flop = 2.0 * 512 * cfg.n_medusa * (cfg.d * cfg.d + cfg.vocab * cfg.d)
    print(json.dumps({"heads_flop": flop, "rows": 512}), flush=True)


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
    from speculative_decoding_heads_amd.model import Model, State, StepGraph, prefill, step, step_workspace_size
    from workloads import TWO_HEAD_CHOICES, TinyConfig, prompt_tokens, tiny_model
    params, heads = tiny_model(0)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    P = dict(params)
    P["embed"], P["final_norm"], P["lm_head"] = up(params["embed"]), up(params["final_norm"]), up(params["lm_head"])
    P["layers"] = [{k: up(v) for k, v in l.items()} for l in params["layers"]]
    model = Model(P, {k: up(v) for k, v in heads.items()}, max_pos=512)
    tree = api.Tree(TWO_HEAD_CHOICES)
    prompt = up(prompt_tokens(100, 1, TinyConfig.prompt_len, TinyConfig.vocab).astype(np.int32))
    st = State(model, 1, 256, 8 * steps)
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
    # the same decoding continued by replays of the step captured once (the state advances
    # with every replay: each replay is the next step)
    gs = torch.cuda.Stream()
    g = StepGraph(model, tree, st, GREEDY, L_hint=256, ws=ws, stream=gs)
    with torch.cuda.stream(gs):
        g.replay(gs)
        torch.cuda.synchronize()
        with Timer() as tg:
            for _ in range(steps):
                g.replay(gs)
        gus = tg.ms() / steps * 1e3
    torch.cuda.synchronize()
    assert int(st.err[0]) == 0
    g.close()
    best = min(us, gus)
    return {"us_per_step": round(best, 2), "steps_per_s": round(1e6 / best, 1),
            "eager_us_per_step": round(us, 2), "graph_us_per_step": round(gus, 2),
            "accepted_tokens_per_step": round(toks, 3), "tok_per_s": round(1e6 / best * toks, 1),
            "bound": "launch latency"}


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


def cpu_baseline(params, heads, sample_layers, model, cfg, tree, prompt, prefix, dev, gpu):
    """The oracle on the host cores, timed on bounded samples (median of 3 repetitions).

    Headline (the 7B-shaped verify step): the Medusa heads on one hidden state (one of
    the 4 heads, scaled x4), 8 of the 32 decoder layers over the 64 tree tokens at the
    prefix (scaled x4), the LM head and typical acceptance, median of 5; matrix products in float32
    BLAS, norms, softmax and the rest in float64.  `oracle_by_config` adds the oracle's
    time for each of the other workloads next to the GPU's (float64 throughout):
    the tiny fp32 step, the attention at batch 1 / prefix 1024, the heads + top-10 +
    candidates at batch 1 (one head scaled x4), the attention at batch 8 / prefix 65536
    (one of its 64 (sequence, KV head) slices, scaled x64) and its compaction."""
    from oracle.attention import attention_slice, tree_attention as oracle_attention
    from oracle.candidates import build_candidates
    from oracle.decoder import forward as oracle_forward
    from oracle.heads import medusa_heads_topk
    from oracle.posterior import GREEDY, TYPICAL, evaluate_posterior_one
    from oracle.tree import tree_buffers
    from oracle.update import kv_compact as oracle_compact
    from workloads import TWO_HEAD_CHOICES, TinyConfig, attention_inputs, seeded_tree_choices, tiny_model
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
    W1, W2 = f32(model.W1[:1]), f32(model.W2[:1])
    H = model.W1.shape[0]
    ot = tree_buffers(seeded_tree_choices(0), K=10)
    rng = np.random.default_rng(0)
    T = ot["T"]
    Hkv, Dh = cfg.n_kv_heads, cfg.head_dim
    Kc = rng.standard_normal((nl, 1, Hkv, prefix, Dh)).astype(np.float32)
    Vc = rng.standard_normal((nl, 1, Hkv, prefix, Dh)).astype(np.float32)
    toks = rng.integers(0, cfg.vocab, (1, T))
    pos = prefix + ot["depth"][None, :]
    h = rng.standard_normal((1, cfg.d)).astype(np.float32)
    med = lambda xs: float(np.median(xs))

    def timed(f):
        t0 = time.perf_counter()
        r = f()
        return time.perf_counter() - t0, r

    log("cpu baseline: timing the oracle")
    per_steps, total = [], 0.0
    for rep in range(5):
        t_heads, _ = timed(lambda: medusa_heads_topk(h, W1, W2, 10, bf16=True))
        t_fwd, (lg, hh, _, _) = timed(lambda: oracle_forward(p, toks, pos, Kc, Vc, np.array([prefix]), ot["anc"],
                                                             bf16=True, mm_dtype=np.float32, layers=nl))
        t_post, _ = timed(lambda: evaluate_posterior_one(ot, lg[0], toks[0], TYPICAL, 0.7, 0.09, 0.3))
        t_lm, _ = timed(lambda: hh[0].astype(np.float32) @ p["lm_head"].T)  # the LM head's share of t_fwd
        per_steps.append(t_heads * H + (t_fwd - t_lm) * (cfg.n_layers / nl) + t_lm + t_post)
        total += t_heads + t_fwd + t_post + t_lm
        log("cpu baseline rep %d: %.2f s per step" % (rep, per_steps[-1]))
    per_step = med(per_steps)

    # ---- the oracle on the other workloads
    by_cfg = {}
    tp, th = tiny_model(0)
    tt = tree_buffers(TWO_HEAD_CHOICES)
    tK = rng.standard_normal((2, 1, 4, 64, 16))
    tV = rng.standard_normal((2, 1, 4, 64, 16))
    ttok = rng.integers(0, TinyConfig.vocab, (1, tt["T"]))
    tpos = 40 + tt["depth"][None, :]
    th_in = rng.standard_normal((1, 64))

    def tiny_step():
        medusa_heads_topk(th_in, th["W1"], th["W2"], tt["K"])
        lg_, _, _, _ = oracle_forward(tp, ttok, tpos, tK, tV, np.array([40]), tt["anc"])
        evaluate_posterior_one(tt, lg_[0], ttok[0], GREEDY)

    ts = [timed(tiny_step)[0] for _ in range(3)]
    by_cfg["tiny_fp32_step"] = {"oracle_us_per_step": round(med(ts) * 1e6, 1), "gpu_us_per_step": gpu["tiny_us"],
                                "sample": "one step: heads, 2-layer forward over the 9 tree tokens, acceptance"}
    q, Kc2, Vc2, Kt2, Vt2, seq2 = attention_inputs(3, 1, T, 32, 8, 128, 1024, 1024, bf16=True)
    ts = [timed(lambda: oracle_attention(q, Kc2, Vc2, seq2, Kt2, Vt2, ot["anc"], 128 ** -0.5))[0] for _ in range(3)]
    by_cfg["tree_attention_B1_L1024"] = {"oracle_us": round(med(ts) * 1e6, 1), "gpu_us": gpu["attn_b1_us"],
                                         "sample": "the whole call (32/8 heads x 128, 64-node tree)"}
    hb = rng.standard_normal((1, cfg.d))
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        tk1, _ = medusa_heads_topk(hb, W1, W2, 10, bf16=True)
        build_candidates(ot, np.zeros(1, np.int64), np.repeat(tk1, H, axis=1), np.array([prefix]))
        ts.append((time.perf_counter() - t0) * H)
    by_cfg["heads_topk_candidates_B1"] = {"oracle_us": round(med(ts) * 1e6, 1), "gpu_us": gpu["heads_b1_us"],
                                          "sample": "one of the 4 heads (d 4096, V 32000, top-10) scaled x4, "
                                                    "plus the candidate expansion"}
    L5 = 65536
    qs = rng.standard_normal((T, 4, Dh))
    Ks5 = rng.standard_normal((L5, Dh)).astype(np.float32)
    Vs5 = rng.standard_normal((L5, Dh)).astype(np.float32)
    Kt5 = rng.standard_normal((T, Dh))
    ts = [timed(lambda: attention_slice(qs, Ks5, Vs5, Kt5, Kt5, ot["anc"], 128 ** -0.5))[0] * 64 for _ in range(3)]
    by_cfg["tree_attention_B8_L65536"] = {"oracle_us": round(med(ts) * 1e6, 1), "gpu_us": gpu["attn_b8_us"],
                                          "sample": "one (sequence, KV head) slice of the 64, scaled x64"}
    cK = np.zeros((1, 8, 8, 200, Dh))
    sK = rng.standard_normal((1, 8, 8, T, Dh))
    bestc = np.zeros(8, np.int64)
    accc = np.minimum(np.arange(8) % 5, ot["path_len"][0] - 1)
    ts = [timed(lambda: oracle_compact(ot, cK, cK, sK, sK, bestc, accc, np.full(8, 100)))[0] for _ in range(3)]
    by_cfg["kv_compact_B8_1layer"] = {"oracle_us": round(med(ts) * 1e6, 1), "gpu_us": gpu["compact_us"],
                                      "sample": "the whole call (cache rows beyond 200 do not change the work)"}
    log("cpu baseline: %.1f s of headline oracle work, median %.2f s per step" % (total, per_step))
    return {"value": round(1.0 / per_step, 5), "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": "heads on one hidden state (1 of %d heads, scaled x%d) + %d of %d decoder layers over the 64 "
                      "tree tokens at prefix %d (scaled x%d) + LM head + typical acceptance; float32 BLAS matrix "
                      "products, float64 elsewhere; median of 5 repetitions (%.1f s measured)"
                      % (H, H, nl, cfg.n_layers, prefix, cfg.n_layers // nl, total),
            "oracle_by_config": by_cfg}


if __name__ == "__main__":
    main()
