"""The library's host C++ -- the static-tree builder and the tree calibration search --
built with AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the device
code is compiled as usual; nothing runs on a GPU) and driven over the same cases as the
CPU ABI tests, valid and invalid: every run must finish clean and give the oracle's
results.  Needs hipcc (the build takes about half a minute)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.calib import best_tree, expected_accept_length
from oracle.tree import anc_bits, tree_buffers
from workloads import PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, chain_choices, seeded_tree_choices

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_heads_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

TREES = [PAGE_TREE_CHOICES, TWO_HEAD_CHOICES, seeded_tree_choices(0), seeded_tree_choices(4), chain_choices(63), []]
BAD_TREES = [([(0,), (0,)], -1), ([(0, 1)], -1), ([(-1,)], -1), ([(k,) for k in range(64)], -2)]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asan") / "host_driver")
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "tree.hip"), os.path.join(CSRC, "calib.hip"),
           os.path.join(ROOT, "tests", "sanitize_host_driver.cpp"), "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-4000:]
    return out


def _run(driver, text):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([driver], input=text, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout.splitlines()


def _tree_line(choices, K=0):
    parts = ["tree", str(K), str(len(choices))]
    for c in choices:
        parts += [str(len(c))] + [str(r) for r in c]
    return " ".join(parts)


def test_tree_builder_under_sanitizers(driver):
    lines = [_tree_line(c) for c in TREES] + [_tree_line(b) for b, _ in BAD_TREES] + [_tree_line([(0,), (3,)], K=3)]
    out = _run(driver, "\n".join(lines) + "\n")
    assert len(out) == len(lines)
    for choices, line in zip(TREES, out):
        f = line.split()
        assert f[0] == "ok", line
        T, D, P = int(f[2]), int(f[4]), int(f[6])
        i = f.index("ti")
        ti = [int(x) for x in f[i + 1:i + 1 + T]]
        i = f.index("parent")
        parent = [int(x) for x in f[i + 1:i + 1 + T]]
        i = f.index("anc")
        anc = [int(x) for x in f[i + 1:i + 1 + T]]
        i = f.index("retrieve")
        ret = np.array([int(x) for x in f[i + 1:]]).reshape(P, D + 1)
        if not choices:
            assert (T, P, D) == (1, 1, 0) and anc == [1]
            continue
        t = tree_buffers(choices)
        assert (T, D, P) == (t["T"], t["D"], t["P"])
        assert ti == t["tree_indices"].tolist() and parent == t["parent"].tolist()
        assert anc == [int(x) for x in anc_bits(t["anc"])]
        assert ret.tolist() == t["retrieve"].tolist()
    codes = [int(l.split()[1]) for l in out[len(TREES):]]
    assert codes == [c for _, c in BAD_TREES] + [-1]


def test_calibration_search_under_sanitizers(driver):
    rng = np.random.default_rng(0)
    cases = []
    for H, K, n in [(4, 10, 64), (5, 8, 48), (1, 10, 11), (3, 3, 40), (4, 10, 1), (2, 2, 7)]:
        a = rng.random((H, K)) ** 3
        a = a / a.sum(1, keepdims=True) * rng.uniform(0.3, 0.95, (H, 1))
        cases.append((a, n))
    ties = rng.integers(1, 4, (3, 4)).astype(np.float64) / 16.0
    cases.append((ties, 50))
    lines = ["accept %d %d %d %s" % (a.shape[0], a.shape[1], n, " ".join("%.17g" % v for v in a.ravel()))
             for a, n in cases]
    bad = ["accept 2 2 3 0.5 0.6 0.1 0.1",   # a depth summing above 1
           "accept 2 2 9 0.5 0.4 0.1 0.1",   # more nodes than the full tree holds
           "accept 2 2 2 -0.1 0.4 0.1 0.1"]  # a negative rate
    out = _run(driver, "\n".join(lines + bad) + "\n")
    for (a, n), line in zip(cases, out):
        f = line.split("|")
        head = f[0].split()
        assert head[0] == "ok", line
        got = [tuple(int(x) for x in seg.split()) for seg in f[1:]]
        want = best_tree(a, n)
        assert got == want
        assert float(head[1]) == expected_accept_length(want, a)
    assert [l.split() for l in out[len(cases):]] == [["status", "-1"]] * 3
