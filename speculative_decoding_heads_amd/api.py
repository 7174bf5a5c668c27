"""Python names of the C ABI calls (same names, torch tensors in, kernels do the work).

Each function takes device tensors, checks their shapes against the call's
layout, and forwards pointers plus the current torch stream to libmedusa.
Outputs are allocated when not supplied.  No arithmetic of the method happens
here.
"""
import ctypes as C

import numpy as np

from . import _lib as L
from ._lib import MedusaError, check, dtype_code, lib, ptr, stream_ptr


def _torch():
    import torch
    return torch


class Tree:
    """A static tree (medusa_tree handle) built from rank-path choices on the current device."""

    def __init__(self, choices, K=None):
        ranks, offsets = [], [0]
        for c in choices:
            ranks.extend(int(r) for r in c)
            offsets.append(len(ranks))
        r = np.asarray(ranks if ranks else [0], dtype=np.int32)
        o = np.asarray(offsets, dtype=np.int32)
        h = C.c_void_p()
        check(lib().medusa_tree_create(r.ctypes.data, o.ctypes.data, len(choices), int(K or 0), C.byref(h)))
        self._h = h
        info = L.TreeHost()
        check(lib().medusa_tree_info(h, C.byref(info)))
        self.T, self.D, self.P, self.K = info.T, info.D, info.P, info.K
        T, P, D = self.T, self.P, self.D
        self.tree_indices = np.array(info.tree_indices[:T], dtype=np.int64)
        self.depth = np.array(info.depth[:T], dtype=np.int64)
        self.parent = np.array(info.parent[:T], dtype=np.int64)
        self.anc_bits = np.array(info.anc[:T], dtype=np.uint64)
        rt = np.array(info.retrieve, dtype=np.int64).reshape(L.MAX_TREE, L.MAX_TREE)
        self.retrieve = rt[:P, : D + 1].copy()
        self.path_len = np.array(info.path_len[:P], dtype=np.int64)

    @property
    def handle(self):
        return self._h

    @property
    def anc_device(self):
        """Device address of the tree's uint64 mask words."""
        return lib().medusa_tree_anc_device(self._h)

    def close(self):
        if self._h:
            check(lib().medusa_tree_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def medusa_heads_topk(h, W1, W2, K, topk_idx=None, topk_val=None, ws=None):
    """h [B, d], W1 [H, d, d], W2 [H, V, d] -> (topk_idx [B, H, K] int32, topk_val [B, H, K] fp32)."""
    torch = _torch()
    B, d = h.shape
    H, V = W2.shape[0], W2.shape[1]
    if W1.shape != (H, d, d) or W2.shape != (H, V, d) or W1.dtype != h.dtype or W2.dtype != h.dtype:
        raise MedusaError("medusa_heads_topk: shape/dtype mismatch")
    dt = dtype_code(h)
    if topk_idx is None:
        topk_idx = torch.empty((B, H, K), dtype=torch.int32, device=h.device)
    if topk_val is None:
        topk_val = torch.empty((B, H, K), dtype=torch.float32, device=h.device)
    need = lib().medusa_heads_topk_workspace_size(dt, B, d, V, H, K)
    ws = L._ws(ws, need, h.device)
    check(lib().medusa_heads_topk(dt, B, d, V, H, K, ptr(h), ptr(W1), ptr(W2), ptr(topk_idx), ptr(topk_val),
                                  ptr(ws), ws.numel(), stream_ptr()))
    return topk_idx, topk_val


def tree_build_candidates(tree, root, topk_idx, seq_len, tree_tokens=None, tree_pos=None, cart=None):
    """root [B], topk_idx [B, H, K], seq_len [B] (int32) -> (tree_tokens [B,T], tree_pos [B,T], cart [B,P,D+1])."""
    torch = _torch()
    B, H, K = topk_idx.shape
    dev = topk_idx.device
    mk = lambda shape: torch.empty(shape, dtype=torch.int32, device=dev)
    tree_tokens = mk((B, tree.T)) if tree_tokens is None else tree_tokens
    tree_pos = mk((B, tree.T)) if tree_pos is None else tree_pos
    cart = mk((B, tree.P, tree.D + 1)) if cart is None else cart
    for t in (root, topk_idx, seq_len):
        if t.dtype != torch.int32:
            raise MedusaError("tree_build_candidates: int32 tensors expected")
    check(lib().tree_build_candidates(tree.handle, B, H, K, ptr(root), ptr(topk_idx), ptr(seq_len), ptr(tree_tokens),
                                      ptr(tree_pos), ptr(cart), stream_ptr()))
    return tree_tokens, tree_pos, cart


def tree_attention_workspace_size(dtype, B, T, Hq, Hkv, Dh, L_hint):
    return lib().tree_attention_workspace_size(dtype, B, T, Hq, Hkv, Dh, int(L_hint))


def tree_attention(q, Kc, Vc, seq_len, Kt, Vt, anc, scale, L_hint=None, out=None, ws=None):
    """q [B,T,Hq,Dh], Kc/Vc [B,Hkv,Lmax,Dh], Kt/Vt [B,Hkv,T,Dh], anc: Tree or int64 device tensor [T]."""
    torch = _torch()
    B, T, Hq, Dh = q.shape
    Hkv, Lmax = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, Hkv, Lmax, Dh) or Vc.shape != Kc.shape or Kt.shape != (B, Hkv, T, Dh) or Vt.shape != Kt.shape:
        raise MedusaError("tree_attention: shape mismatch")
    if seq_len.dtype != torch.int32:
        raise MedusaError("tree_attention: seq_len must be int32")
    dt = dtype_code(q)
    L_hint = Lmax if L_hint is None else int(L_hint)
    if out is None:
        out = torch.empty_like(q)
    anc_p = anc.anc_device if isinstance(anc, Tree) else ptr(anc)
    need = lib().tree_attention_workspace_size(dt, B, T, Hq, Hkv, Dh, L_hint)
    ws = L._ws(ws, need, q.device)
    check(lib().tree_attention(dt, B, T, Hq, Hkv, Dh, ptr(q), ptr(Kc), ptr(Vc), Lmax, L_hint, ptr(seq_len), ptr(Kt),
                               ptr(Vt), anc_p, float(scale), ptr(out), ptr(ws), ws.numel(), stream_ptr()))
    return out


def tree_attention_noalloc(q, Kc, Vc, seq_len, Kt, Vt, anc, scale, L_hint=None, out=None):
    """tree_attention with the split partials in the library's fixed scratch (no workspace)."""
    torch = _torch()
    B, T, Hq, Dh = q.shape
    Hkv, Lmax = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, Hkv, Lmax, Dh) or Vc.shape != Kc.shape or Kt.shape != (B, Hkv, T, Dh) or Vt.shape != Kt.shape:
        raise MedusaError("tree_attention_noalloc: shape mismatch")
    if seq_len.dtype != torch.int32:
        raise MedusaError("tree_attention_noalloc: seq_len must be int32")
    L_hint = Lmax if L_hint is None else int(L_hint)
    if out is None:
        out = torch.empty_like(q)
    anc_p = anc.anc_device if isinstance(anc, Tree) else ptr(anc)
    check(lib().tree_attention_noalloc(dtype_code(q), B, T, Hq, Hkv, Dh, ptr(q), ptr(Kc), ptr(Vc), Lmax, L_hint,
                                       ptr(seq_len), ptr(Kt), ptr(Vt), anc_p, float(scale), ptr(out), stream_ptr()))
    return out


def evaluate_posterior(tree, logits, tree_tokens, mode, temperature=0.0, eps=0.09, delta=0.3, outs=None, ws=None):
    """logits [B,T,V] fp32, tree_tokens [B,T] int32 -> (best, accept_len, sel_node, next_root) int32 [B]."""
    torch = _torch()
    B, T, V = logits.shape
    if T != tree.T or logits.dtype != torch.float32:
        raise MedusaError("evaluate_posterior: logits must be fp32 [B, T, V] with T = tree nodes")
    if outs is None:
        outs = [torch.empty(B, dtype=torch.int32, device=logits.device) for _ in range(4)]
    need = lib().evaluate_posterior_workspace_size(B, T)
    ws = L._ws(ws, need, logits.device)
    check(lib().evaluate_posterior(tree.handle, B, V, ptr(logits), ptr(tree_tokens), int(mode), float(temperature),
                                   float(eps), float(delta), *[ptr(o) for o in outs], ptr(ws), ws.numel(),
                                   stream_ptr()))
    return tuple(outs)


def sample_tokens(logits, sampling, pos, seq_id=None, out=None):
    """medusa_sample_tokens: logits [M, V] fp32, pos [M] int32 (and seq_id [M] int32 or row index)
    -> tokens [M] int32.  sampling: dict(kind, temperature, eps, delta, top_p, seed)."""
    torch = _torch()
    M, V = logits.shape
    if logits.dtype != torch.float32 or pos.dtype != torch.int32 or pos.numel() != M:
        raise MedusaError("sample_tokens: fp32 logits [M, V] and int32 positions [M] expected")
    out = torch.empty(M, dtype=torch.int32, device=logits.device) if out is None else out
    sd = L.sampling_desc(sampling)
    check(lib().medusa_sample_tokens(C.byref(sd), M, V, ptr(logits), logits.stride(0), ptr(seq_id), ptr(pos),
                                     ptr(out), stream_ptr()))
    return out


def evaluate_posterior_sampled(tree, logits, tree_tokens, tree_pos, sampling, outs=None, ws=None):
    """Non-fast acceptance: logits [B,T,V] fp32, tree_tokens / tree_pos [B,T] int32
    -> (best, accept_len, sel_node, next_root) int32 [B]."""
    torch = _torch()
    B, T, V = logits.shape
    if T != tree.T or logits.dtype != torch.float32:
        raise MedusaError("evaluate_posterior_sampled: logits must be fp32 [B, T, V] with T = tree nodes")
    if outs is None:
        outs = [torch.empty(B, dtype=torch.int32, device=logits.device) for _ in range(4)]
    ws = L._ws(ws, lib().evaluate_posterior_sampled_workspace_size(B, T), logits.device)
    sd = L.sampling_desc(sampling)
    check(lib().evaluate_posterior_sampled(tree.handle, B, V, ptr(logits), ptr(tree_tokens), ptr(tree_pos),
                                           C.byref(sd), *[ptr(o) for o in outs], ptr(ws), ws.numel(), stream_ptr()))
    return tuple(outs)


def kv_compact(tree, Kc, Vc, Kt, Vt, best, accept_len, seq_len, tree_tokens, out_tokens=None, n_out=None,
               err_flag=None):
    """Kc/Vc [NL,B,Hkv,Lmax,Dh], Kt/Vt [NL,B,Hkv,T,Dh]; updates Kc, Vc, seq_len, out_tokens, n_out in place."""
    NL, B, Hkv, Lmax, Dh = Kc.shape
    if Kt.shape != (NL, B, Hkv, tree.T, Dh):
        raise MedusaError("kv_compact: side buffer shape mismatch")
    max_new = out_tokens.shape[1] if out_tokens is not None else 0
    check(lib().kv_compact(dtype_code(Kc), tree.handle, NL, B, Hkv, Dh, Lmax, ptr(Kc), ptr(Vc), ptr(Kt), ptr(Vt),
                           ptr(best), ptr(accept_len), ptr(seq_len), ptr(tree_tokens), ptr(out_tokens), max_new,
                           ptr(n_out), ptr(err_flag), stream_ptr()))


# ---- decoder building blocks ------------------------------------------------
def gemm(A, W, epilogue=L.EPI_F32, out=None, R=None, ws=None):
    """A [M, K], W [N, K] -> epilogue(A W^T)."""
    torch = _torch()
    M, K = A.shape
    N = W.shape[0]
    dt = dtype_code(A)
    if out is None:
        if epilogue == L.EPI_F32:
            out = torch.empty((M, N), dtype=torch.float32, device=A.device)
        elif epilogue == L.EPI_SWIGLU:
            out = torch.empty((M, N // 2), dtype=A.dtype, device=A.device)
        else:
            out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    ldc = out.shape[-1]
    need = lib().medusa_gemm_workspace_size(dt, M, N, K, 1)
    ws = L._ws(ws, need, A.device)
    check(lib().medusa_gemm(dt, M, N, K, ptr(A), K, 0, ptr(W), 0, ptr(out), ldc, 0, 1, int(epilogue), ptr(R),
                            R.shape[-1] if R is not None else 0, 0, ptr(ws), ws.numel(), stream_ptr()))
    return out


def rmsnorm(x, w, eps, out=None):
    out = _torch().empty_like(x) if out is None else out
    M, N = x.shape
    check(lib().medusa_rmsnorm(dtype_code(x), M, N, ptr(x), ptr(w), float(eps), ptr(out), stream_ptr()))
    return out


def gemm_resid_rmsnorm(A, W, X, norm_w, eps, Y=None, ws=None):
    """X += A W^T in place, then Y = RMSNorm(X) * norm_w; returns Y."""
    M, K = A.shape
    N = W.shape[0]
    Y = _torch().empty_like(X) if Y is None else Y
    need = lib().medusa_gemm_resid_rmsnorm_workspace_size(dtype_code(A), M, N, K)
    ws = L._ws(ws, need, A.device)
    check(lib().medusa_gemm_resid_rmsnorm(dtype_code(A), M, N, K, ptr(A), A.stride(0), ptr(W), ptr(X), ptr(norm_w),
                                          float(eps), ptr(Y), ptr(ws), ws.numel(), stream_ptr()))
    return Y


def argmax_rows(x, out=None):
    torch = _torch()
    M, V = x.shape
    out = torch.empty(M, dtype=torch.int32, device=x.device) if out is None else out
    check(lib().medusa_argmax_rows(M, V, ptr(x), V, ptr(out), stream_ptr()))
    return out


def topk_rows(x, K):
    torch = _torch()
    M, V = x.shape
    idx = torch.empty((M, K), dtype=torch.int32, device=x.device)
    val = torch.empty((M, K), dtype=torch.float32, device=x.device)
    ws = L._ws(None, lib().medusa_topk_rows_workspace_size(M, V, K), x.device)
    check(lib().medusa_topk_rows(M, V, ptr(x), K, ptr(idx), ptr(val), ptr(ws), ws.numel(), stream_ptr()))
    return idx, val


def tree_from_acceptance(acc, n_nodes):
    """medusa_tree_from_acceptance: (choices in selection order, expected accepted length).

    acc: [H, K] per-(depth, rank) acceptance rates (host array); host-only call."""
    a = np.ascontiguousarray(np.asarray(acc, dtype=np.float64))
    if a.ndim != 2:
        raise L.MedusaError("tree_from_acceptance: acc must be [H, K]")
    H, K = a.shape
    n = int(n_nodes)
    ranks = np.zeros(max(n - 1, 1) * H, np.int32)
    offsets = np.zeros(max(n, 1), np.int32)
    exp = C.c_double(0.0)
    check(lib().medusa_tree_from_acceptance(a.ctypes.data, H, K, n, ranks.ctypes.data, offsets.ctypes.data,
                                            C.byref(exp)))
    choices = [tuple(int(r) for r in ranks[offsets[i]:offsets[i + 1]]) for i in range(n - 1)]
    return choices, exp.value


def head_hits(topk, tokens, counts=None, positions=None):
    """medusa_head_hits on device tensors: topk [N, H, K] int32, tokens [n] int32.

    Adds to counts [H, K] / positions [H] (int64, zeroed here when not given)."""
    torch = _torch()
    N, H, K = topk.shape
    if counts is None:
        counts = torch.zeros((H, K), dtype=torch.int64, device=topk.device)
    if positions is None:
        positions = torch.zeros(H, dtype=torch.int64, device=topk.device)
    check(lib().medusa_head_hits(N, H, K, ptr(topk), ptr(tokens), tokens.numel(), ptr(counts), ptr(positions),
                                 stream_ptr()))
    return counts, positions
