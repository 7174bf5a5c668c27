"""Model / state wrappers around medusa_forward, medusa_prefill and medusa_step.

Weights arrive as torch device tensors in the per-matrix layout of a LLaMA-style
decoder (wq, wk, wv, wo, w_gate, w_up, w_down, norms, embedding, LM head) plus
the Medusa heads (W1 [H, d, d], W2 [H, V, d]).  At load time they are packed
into the library's layout: Q/K/V rows stacked into one matrix, gate and up rows
interleaved (row 2j = gate j, row 2j+1 = up j).  The rotary tables are computed
once on the host in float64 and stored as float32 device tables.
"""
import ctypes as C

import numpy as np

from . import _lib as L
from ._lib import MedusaError, check, dtype_code, lib, ptr, stream_ptr


def _torch():
    import torch
    return torch


def rope_tables(max_pos, head_dim, theta, device):
    torch = _torch()
    half = head_dim // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    cos = torch.from_numpy(np.cos(ang).astype(np.float32)).to(device)
    sin = torch.from_numpy(np.sin(ang).astype(np.float32)).to(device)
    return cos, sin


class Model:
    """Holds packed device weights and the medusa_model descriptor."""

    def __init__(self, params, heads, max_pos, device=None):
        torch = _torch()
        emb = params["embed"]
        device = emb.device if device is None else device
        self.dtype = emb.dtype
        self.keep = []
        layers = params["layers"]
        NL = len(layers)
        d = emb.shape[1]
        self.d, self.V = d, emb.shape[0]
        self.Hq, self.Hkv, self.Dh = params["n_heads"], params["n_kv_heads"], params["head_dim"]
        self.F = layers[0]["w_gate"].shape[0]
        self.NL = NL
        self.H = heads["W1"].shape[0] if heads is not None else 0
        self.eps = float(params["norm_eps"])
        lw = (L.LayerWeights * NL)()
        for i, p in enumerate(layers):
            wqkv = torch.cat([p["wq"], p["wk"], p["wv"]], dim=0).contiguous()
            wgu = torch.stack([p["w_gate"], p["w_up"]], dim=1).reshape(2 * self.F, d).contiguous()
            an, fn = p["attn_norm"].contiguous(), p["ffn_norm"].contiguous()
            wo, wd = p["wo"].contiguous(), p["w_down"].contiguous()
            self.keep += [wqkv, wgu, an, fn, wo, wd]
            lw[i] = L.LayerWeights(ptr(an), ptr(wqkv), ptr(wo), ptr(fn), ptr(wgu), ptr(wd))
        self.layer_array = lw
        self.cos, self.sin = rope_tables(max_pos, self.Dh, params["rope_theta"], device)
        self.final_norm = params["final_norm"].contiguous()
        self.lm_head = params["lm_head"].contiguous()
        self.embed = emb.contiguous()
        self.keep += [self.cos, self.sin, self.final_norm, self.lm_head, self.embed]
        w1 = heads["W1"].contiguous() if heads is not None else None
        w2 = heads["W2"].contiguous() if heads is not None else None
        self.W1, self.W2 = w1, w2
        self.desc = L.ModelDesc(
            dtype_code(emb), NL, d, self.Hq, self.Hkv, self.Dh, self.F, self.V, self.eps, ptr(self.embed),
            ptr(self.final_norm), ptr(self.lm_head), C.cast(lw, C.POINTER(L.LayerWeights)), ptr(self.cos),
            ptr(self.sin), max_pos, self.H, ptr(w1) if w1 is not None else None, ptr(w2) if w2 is not None else None)
        self.device = device

    def forward_workspace_size(self, B, T, L_hint):
        return lib().medusa_forward_workspace_size(C.byref(self.desc), B, T, int(L_hint))

    def trace_buffers(self, B, T):
        """Device buffers for forward(..., trace=...): each stage's output of every layer."""
        torch = _torch()
        M, dev, dt = B * T, self.device, self.dtype
        e = lambda *s: torch.empty(s, dtype=dt, device=dev)
        return dict(x=e(self.NL + 1, M, self.d), xn=e(self.NL, M, self.d), q=e(self.NL, M, self.Hq * self.Dh),
                    attn=e(self.NL, M, self.Hq * self.Dh), x_mid=e(self.NL, M, self.d), act=e(self.NL, M, self.F))

    def forward(self, tokens, pos, Kc, Vc, seq_len, anc, L_hint=None, Kt=None, Vt=None, ws=None, trace=None):
        """tokens, pos [B, T] int32; Kc/Vc [NL, B, Hkv, Lmax, Dh] -> (logits [B,T,V], h [B,T,d], Kt, Vt).

        trace: optional dict of device buffers (trace_buffers(B, T)) that receive each
        stage's output of every layer (medusa_forward_trace)."""
        torch = _torch()
        B, T = tokens.shape
        Lmax = Kc.shape[3] if Kc is not None else 0
        L_hint = Lmax if L_hint is None else int(L_hint)
        dev = tokens.device
        if Kt is None:
            Kt = torch.empty((self.NL, B, self.Hkv, T, self.Dh), dtype=self.dtype, device=dev)
            Vt = torch.empty_like(Kt)
        logits = torch.empty((B, T, self.V), dtype=torch.float32, device=dev)
        h = torch.empty((B, T, self.d), dtype=self.dtype, device=dev)
        ws = L._ws(ws, self.forward_workspace_size(B, T, L_hint), dev)
        anc_p = anc.anc_device if hasattr(anc, "anc_device") else ptr(anc)
        if trace is not None:
            M = B * T
            shapes = dict(x=(self.NL + 1, M, self.d), xn=(self.NL, M, self.d), q=(self.NL, M, self.Hq * self.Dh),
                          attn=(self.NL, M, self.Hq * self.Dh), x_mid=(self.NL, M, self.d), act=(self.NL, M, self.F))
            for k, v in trace.items():
                if k not in shapes or tuple(v.shape) != shapes[k] or v.dtype != self.dtype:
                    raise MedusaError("forward: trace buffer %s must be %s %s" % (k, shapes.get(k), self.dtype))
            td = L.TraceDesc(*[ptr(trace.get(k)) for k in ("x", "xn", "q", "attn", "x_mid", "act")])
            check(lib().medusa_forward_trace(C.byref(self.desc), B, T, ptr(tokens), ptr(pos), ptr(Kc), ptr(Vc), Lmax,
                                             L_hint, ptr(seq_len), ptr(Kt), ptr(Vt), anc_p, ptr(logits), ptr(h),
                                             C.byref(td), ptr(ws), ws.numel(), stream_ptr()))
        else:
            check(lib().medusa_forward(C.byref(self.desc), B, T, ptr(tokens), ptr(pos), ptr(Kc), ptr(Vc), Lmax,
                                       L_hint, ptr(seq_len), ptr(Kt), ptr(Vt), anc_p, ptr(logits), ptr(h), ptr(ws),
                                       ws.numel(), stream_ptr()))
        return logits, h, Kt, Vt


class State:
    """Device buffers of B sequences in generation (medusa_state)."""

    def __init__(self, model, B, Lmax, max_new, stop_token=None, sampling=None):
        """stop_token: per-sequence stop (an int >= 0, or -1 for output/cache room only);
        None keeps the plain behaviour (every step appends all accepted tokens).
        sampling: dict(kind, temperature, eps, delta, top_p, seed) for sampled generation
        (the root drawn at prefill and steps with mode SAMPLED); None keeps the argmax root."""
        torch = _torch()
        dev = model.device
        i32 = lambda *s: torch.zeros(s, dtype=torch.int32, device=dev)
        self.B, self.Lmax, self.max_new = B, Lmax, max_new
        self.Kc = torch.zeros((model.NL, B, model.Hkv, Lmax, model.Dh), dtype=model.dtype, device=dev)
        self.Vc = torch.zeros_like(self.Kc)
        self.seq_len, self.root, self.n_out = i32(B), i32(B), i32(B)
        self.h_sel = torch.zeros((B, model.d), dtype=model.dtype, device=dev)
        self.out_tokens = i32(B, max(max_new, 1))
        self.err = i32(1)
        self.best, self.accept_len, self.sel_node = i32(B), i32(B), i32(B)
        self.done = i32(B) if stop_token is not None else None
        self.stop_token = -1 if stop_token is None else int(stop_token)
        self.sampling = L.sampling_desc(sampling) if sampling is not None else None
        self.desc = L.StateDesc(ptr(self.Kc), ptr(self.Vc), Lmax, ptr(self.seq_len), ptr(self.root), ptr(self.h_sel),
                                ptr(self.out_tokens), max_new, ptr(self.n_out), ptr(self.err), ptr(self.best),
                                ptr(self.accept_len), ptr(self.sel_node), ptr(self.done), self.stop_token,
                                C.pointer(self.sampling) if self.sampling is not None else None)


def prefill(model, state, prompt, ws=None):
    """prompt [B, S] int32 device tensor."""
    B, S = prompt.shape
    need = lib().medusa_prefill_workspace_size(C.byref(model.desc), B, S, state.Lmax)
    ws = L._ws(ws, need, prompt.device)
    check(lib().medusa_prefill(C.byref(model.desc), B, S, ptr(prompt), C.byref(state.desc), ptr(ws), ws.numel(),
                               stream_ptr()))


def step_workspace_size(model, tree, B, L_hint):
    return lib().medusa_step_workspace_size(C.byref(model.desc), tree.handle, B, int(L_hint))


class StepGraph:
    """One verify step captured into a HIP graph (medusa_step_graph_create); replay() launches it.

    Capture happens on ``stream`` (a non-default torch stream); every pointer,
    including the state and workspace, is baked into the graph, so keep them alive."""

    def __init__(self, model, tree, state, mode, temperature=0.0, eps=0.09, delta=0.3, L_hint=None, ws=None,
                 stream=None):
        torch = _torch()
        L_hint = state.Lmax if L_hint is None else int(L_hint)
        self.ws = L._ws(ws, step_workspace_size(model, tree, state.B, L_hint), state.Kc.device)
        self.stream = stream or torch.cuda.Stream()
        self.refs = (model, tree, state)
        h = C.c_void_p()
        torch.cuda.synchronize()
        check(lib().medusa_step_graph_create(C.byref(model.desc), tree.handle, state.B, int(mode), float(temperature),
                                             float(eps), float(delta), C.byref(state.desc), L_hint, None,
                                             ptr(self.ws), self.ws.numel(), self.stream.cuda_stream, C.byref(h)))
        self._h = h

    def replay(self, stream=None):
        s = stream if stream is not None else _torch().cuda.current_stream()
        check(lib().medusa_graph_launch(self._h, s.cuda_stream))

    def close(self):
        if getattr(self, "_h", None):
            check(lib().medusa_graph_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def step(model, tree, state, mode, temperature=0.0, eps=0.09, delta=0.3, L_hint=None, topk_override=None, ws=None):
    B = state.B
    L_hint = state.Lmax if L_hint is None else int(L_hint)
    ws = L._ws(ws, step_workspace_size(model, tree, B, L_hint), state.Kc.device)
    check(lib().medusa_step(C.byref(model.desc), tree.handle, B, int(mode), float(temperature), float(eps),
                            float(delta), C.byref(state.desc), L_hint, ptr(topk_override), ptr(ws), ws.numel(),
                            stream_ptr()))


def step_fused_workspace_size(model, tree, B, L_hint):
    return lib().medusa_step_fused_workspace_size(C.byref(model.desc), tree.handle, B, int(L_hint))


def init_topk_carry(model, tree, state):
    """The first fused step's candidates: the heads' top-K on h_sel (after prefill or a plain step)."""
    from . import api
    idx, _ = api.medusa_heads_topk(state.h_sel, model.W1, model.W2, tree.K)
    return idx


def step_fused(model, tree, state, topk_carry, mode, temperature=0.0, eps=0.09, delta=0.3, L_hint=None, ws=None):
    """medusa_step_fused: heads on every tree node in the step; topk_carry [B, H, K] int32 in and out."""
    B = state.B
    L_hint = state.Lmax if L_hint is None else int(L_hint)
    if tuple(topk_carry.shape) != (B, model.H, tree.K) or str(topk_carry.dtype) != "torch.int32":
        raise L.MedusaError("step_fused: topk_carry must be int32 [B, H, K]")
    ws = L._ws(ws, step_fused_workspace_size(model, tree, B, L_hint), state.Kc.device)
    check(lib().medusa_step_fused(C.byref(model.desc), tree.handle, B, int(mode), float(temperature), float(eps),
                                  float(delta), C.byref(state.desc), ptr(topk_carry), L_hint, ptr(ws), ws.numel(),
                                  stream_ptr()))

