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
