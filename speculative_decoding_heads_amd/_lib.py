"""ctypes binding of libmedusa.so: argument marshalling only.

Every computation runs in the library's HIP kernels; this module converts
torch tensors (device memory) and the current torch stream into the C ABI's
plain pointers, and raises when a call returns an error.  There is no CPU or
PyTorch fallback: if the shared library is missing, loading fails loudly.
"""
import ctypes as C
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmedusa.so")

MEDUSA_F32, MEDUSA_BF16 = 0, 1
GREEDY, TYPICAL, SAMPLED = 0, 1, 2
SAMPLE_TYPICAL, SAMPLE_NUCLEUS = 1, 2
EPI_F32, EPI_STORE, EPI_RESID, EPI_SILU_RESID_A, EPI_SWIGLU = 0, 1, 2, 3, 4
MAX_TREE = 64

EXPORTED = [
    "medusa_last_error", "medusa_version", "medusa_tree_create", "medusa_tree_build_host", "medusa_tree_info",
    "medusa_tree_anc_device",
    "medusa_tree_destroy", "medusa_heads_topk_workspace_size", "medusa_heads_topk", "tree_build_candidates",
    "tree_attention_workspace_size", "tree_attention", "tree_attention_noalloc_max_scratch", "tree_attention_noalloc",
    "evaluate_posterior_workspace_size", "evaluate_posterior",
    "kv_compact", "medusa_gemm_workspace_size", "medusa_gemm", "medusa_rmsnorm",
    "medusa_gemm_resid_rmsnorm_workspace_size", "medusa_gemm_resid_rmsnorm", "medusa_rope_split",
    "medusa_embed", "medusa_gather_rows", "medusa_argmax_rows", "medusa_topk_rows_workspace_size",
    "medusa_topk_rows",
    "medusa_forward_workspace_size", "medusa_forward", "medusa_forward_trace", "medusa_prefill_workspace_size",
    "medusa_prefill",
    "medusa_step_workspace_size", "medusa_step", "medusa_step_graph_create", "medusa_graph_launch",
    "medusa_graph_destroy", "medusa_step_fused_workspace_size", "medusa_step_fused",
    "medusa_tree_from_acceptance", "medusa_head_hits", "medusa_sample_tokens",
    "evaluate_posterior_sampled_workspace_size", "evaluate_posterior_sampled", "medusa_read_probe",
]


class MedusaError(RuntimeError):
    pass


class TreeHost(C.Structure):
    _fields_ = [("T", C.c_int32), ("D", C.c_int32), ("P", C.c_int32), ("K", C.c_int32), ("H", C.c_int32),
                ("tree_indices", C.c_int32 * MAX_TREE), ("depth", C.c_int32 * MAX_TREE),
                ("parent", C.c_int32 * MAX_TREE), ("path_len", C.c_int32 * MAX_TREE),
                ("anc", C.c_uint64 * MAX_TREE), ("retrieve", C.c_int32 * (MAX_TREE * MAX_TREE))]


class LayerWeights(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p), ("wqkv", C.c_void_p), ("wo", C.c_void_p), ("ffn_norm", C.c_void_p),
                ("w_gate_up", C.c_void_p), ("w_down", C.c_void_p)]


class ModelDesc(C.Structure):
    _fields_ = [("dtype", C.c_int), ("n_layers", C.c_int), ("d", C.c_int), ("n_heads", C.c_int),
                ("n_kv_heads", C.c_int), ("head_dim", C.c_int), ("ffn", C.c_int), ("vocab", C.c_int),
                ("norm_eps", C.c_float), ("embed", C.c_void_p), ("final_norm", C.c_void_p),
                ("lm_head", C.c_void_p), ("layers", C.POINTER(LayerWeights)), ("rope_cos", C.c_void_p),
                ("rope_sin", C.c_void_p), ("rope_max_pos", C.c_int), ("n_medusa", C.c_int),
                ("medusa_w1", C.c_void_p), ("medusa_w2", C.c_void_p)]


class TraceDesc(C.Structure):
    _fields_ = [("x", C.c_void_p), ("xn", C.c_void_p), ("q", C.c_void_p), ("attn", C.c_void_p),
                ("x_mid", C.c_void_p), ("act", C.c_void_p)]


class SamplingDesc(C.Structure):
    _fields_ = [("kind", C.c_int32), ("temperature", C.c_float), ("eps", C.c_float), ("delta", C.c_float),
                ("top_p", C.c_float), ("seed", C.c_uint64)]


def sampling_desc(sampling):
    """medusa_sampling from a dict(kind, temperature, eps, delta, top_p, seed)."""
    s = sampling
    return SamplingDesc(int(s["kind"]), float(s["temperature"]), float(s.get("eps", 0.09)),
                        float(s.get("delta", 0.3)), float(s.get("top_p", 0.8)), int(s.get("seed", 0)))


class StateDesc(C.Structure):
    _fields_ = [("Kc", C.c_void_p), ("Vc", C.c_void_p), ("Lmax", C.c_int64), ("seq_len", C.c_void_p),
                ("root", C.c_void_p), ("h_sel", C.c_void_p), ("out_tokens", C.c_void_p), ("max_new", C.c_int),
                ("n_out", C.c_void_p), ("err", C.c_void_p), ("best", C.c_void_p), ("accept_len", C.c_void_p),
                ("sel_node", C.c_void_p), ("done", C.c_void_p), ("stop_token", C.c_int32),
                ("sampling", C.POINTER(SamplingDesc))]


_lib = None

_I, _L, _F, _P, _S = C.c_int, C.c_int64, C.c_float, C.c_void_p, C.c_size_t


def _declare(lib):
    sig = {
        "medusa_last_error": (C.c_char_p, []),
        "medusa_version": (_I, []),
        "medusa_tree_create": (_I, [_P, _P, C.c_int32, C.c_int32, C.POINTER(_P)]),
        "medusa_tree_build_host": (_I, [_P, _P, C.c_int32, C.c_int32, C.POINTER(TreeHost)]),
        "medusa_tree_info": (_I, [_P, C.POINTER(TreeHost)]),
        "medusa_tree_anc_device": (_P, [_P]),
        "medusa_tree_destroy": (_I, [_P]),
        "medusa_heads_topk_workspace_size": (_S, [_I] * 6),
        "medusa_heads_topk": (_I, [_I] * 6 + [_P] * 5 + [_P, _S, _P]),
        "tree_build_candidates": (_I, [_P, _I, _I, _I] + [_P] * 6 + [_P]),
        "tree_attention_workspace_size": (_S, [_I] * 6 + [_L]),
        "tree_attention": (_I, [_I] * 6 + [_P, _P, _P, _L, _L, _P, _P, _P, _P, _F, _P, _P, _S, _P]),
        "tree_attention_noalloc_max_scratch": (_S, []),
        "tree_attention_noalloc": (_I, [_I] * 6 + [_P, _P, _P, _L, _L, _P, _P, _P, _P, _F, _P, _P]),
        "evaluate_posterior_workspace_size": (_S, [_I, _I]),
        "evaluate_posterior": (_I, [_P, _I, _I, _P, _P, _I, _F, _F, _F, _P, _P, _P, _P, _P, _S, _P]),
        "kv_compact": (_I, [_I, _P, _I, _I, _I, _I, _L] + [_P] * 9 + [_I, _P, _P, _P]),
        "medusa_gemm_workspace_size": (_S, [_I] * 5),
        "medusa_gemm": (_I, [_I] * 4 + [_P, _L, _L, _P, _L, _P, _L, _L, _I, _I, _P, _L, _L, _P, _S, _P]),
        "medusa_rmsnorm": (_I, [_I, _I, _I, _P, _P, _F, _P, _P]),
        "medusa_gemm_resid_rmsnorm_workspace_size": (_S, [_I] * 4),
        "medusa_gemm_resid_rmsnorm": (_I, [_I] * 4 + [_P, _L, _P, _P, _P, _F, _P, _P, _S, _P]),
        "medusa_rope_split": (_I, [_I] * 6 + [_P] * 4 + [_I, _P, _P, _P, _P]),
        "medusa_embed": (_I, [_I, _I, _I, _P, _P, _I, _P, _P]),
        "medusa_gather_rows": (_I, [_I, _I, _I, _I, _P, _P, _P, _P]),
        "medusa_argmax_rows": (_I, [_I, _I, _P, _L, _P, _P]),
        "medusa_topk_rows_workspace_size": (_S, [_I, _I, _I]),
        "medusa_topk_rows": (_I, [_I, _I, _P, _I, _P, _P, _P, _S, _P]),
        "medusa_forward_workspace_size": (_S, [C.POINTER(ModelDesc), _I, _I, _L]),
        "medusa_forward": (_I, [C.POINTER(ModelDesc), _I, _I, _P, _P, _P, _P, _L, _L, _P, _P, _P, _P, _P, _P, _P,
                                _S, _P]),
        "medusa_forward_trace": (_I, [C.POINTER(ModelDesc), _I, _I, _P, _P, _P, _P, _L, _L, _P, _P, _P, _P, _P, _P,
                                      C.POINTER(TraceDesc), _P, _S, _P]),
        "medusa_prefill_workspace_size": (_S, [C.POINTER(ModelDesc), _I, _I, _L]),
        "medusa_prefill": (_I, [C.POINTER(ModelDesc), _I, _I, _P, C.POINTER(StateDesc), _P, _S, _P]),
        "medusa_step_workspace_size": (_S, [C.POINTER(ModelDesc), _P, _I, _L]),
        "medusa_step": (_I, [C.POINTER(ModelDesc), _P, _I, _I, _F, _F, _F, C.POINTER(StateDesc), _L, _P, _P, _S,
                             _P]),
        "medusa_step_graph_create": (_I, [C.POINTER(ModelDesc), _P, _I, _I, _F, _F, _F, C.POINTER(StateDesc), _L,
                                          _P, _P, _S, _P, C.POINTER(_P)]),
        "medusa_step_fused_workspace_size": (_S, [C.POINTER(ModelDesc), _P, _I, _L]),
        "medusa_step_fused": (_I, [C.POINTER(ModelDesc), _P, _I, _I, _F, _F, _F, C.POINTER(StateDesc), _P, _L, _P,
                                   _S, _P]),
        "medusa_tree_from_acceptance": (_I, [_P, C.c_int32, C.c_int32, C.c_int32, _P, _P, C.POINTER(C.c_double)]),
        "medusa_head_hits": (_I, [_I, _I, _I, _P, _P, _I, _P, _P, _P]),
        "medusa_sample_tokens": (_I, [C.POINTER(SamplingDesc), _I, _I, _P, _L, _P, _P, _P, _P]),
        "evaluate_posterior_sampled_workspace_size": (_S, [_I, _I]),
        "evaluate_posterior_sampled": (_I, [_P, _I, _I, _P, _P, _P, C.POINTER(SamplingDesc), _P, _P, _P, _P, _P, _S,
                                            _P]),
        "medusa_read_probe": (_I, [_P, _S, _I, _P, _P]),
        "medusa_graph_launch": (_I, [_P, _P]),
        "medusa_graph_destroy": (_I, [_P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args


def lib():
    """The loaded library (raises if libmedusa.so has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MedusaError("libmedusa.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


def check(rc):
    if rc != 0:
        raise MedusaError("libmedusa error %d: %s" % (rc, lib().medusa_last_error().decode()))


# ---------------------------------------------------------------------------
# torch helpers
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return MEDUSA_F32
    if t.dtype == torch.bfloat16:
        return MEDUSA_BF16
    raise MedusaError("unsupported dtype %s" % t.dtype)


def ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise MedusaError("expected a device tensor")
    if not t.is_contiguous():
        raise MedusaError("expected a contiguous tensor")
    return t.data_ptr()


def stream_ptr():
    return _torch().cuda.current_stream().cuda_stream


def workspace(nbytes, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _ws(ws, nbytes, device):
    if ws is None:
        ws = workspace(nbytes, device)
    if ws.numel() < nbytes:
        raise MedusaError("workspace of %d bytes < %d" % (ws.numel(), nbytes))
    return ws
