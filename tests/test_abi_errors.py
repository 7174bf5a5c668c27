"""Argument errors of the five verify-step calls (and the no-allocation attention
entry): each returns its documented status -- MEDUSA_ERR_ARG (-1), _UNSUPPORTED (-2)
or _WORKSPACE (-3) -- with a message naming the problem, and returns before any
device work, so these run on a machine without a GPU.  The checks that need a
built tree (rank stride, tree depth) are in the GPU suite."""
import ctypes as C

import pytest

ARG, UNSUP, WS = -1, -2, -3
P = C.c_void_p
FAKE = P(0x1000)  # a non-null pointer that is never dereferenced on these paths


def _lib():
    from speculative_decoding_heads_amd._lib import lib
    return lib()


def _expect(rc, code, words):
    lib = _lib()
    assert rc == code, (rc, code, lib.medusa_last_error())
    msg = lib.medusa_last_error().decode()
    for w in words:
        assert w in msg, (w, msg)


def _heads(dtype=1, B=1, d=64, V=100, H=2, K=4, ptrs=(FAKE,) * 4, ws=FAKE, ws_bytes=1 << 30):
    h, W1, W2, idx = ptrs
    return _lib().medusa_heads_topk(dtype, B, d, V, H, K, h, W1, W2, idx, None, ws, ws_bytes, None)


def test_heads_topk_errors():
    _expect(_heads(dtype=7), UNSUP, ["dtype"])
    _expect(_heads(d=0), ARG, ["bad sizes"])
    _expect(_heads(K=17), UNSUP, ["K=17"])
    _expect(_heads(K=0), UNSUP, ["K=0"])
    _expect(_heads(d=48), UNSUP, ["d % 32"])
    _expect(_heads(ptrs=(FAKE, None, FAKE, FAKE)), ARG, ["null pointer"])
    need = _lib().medusa_heads_topk_workspace_size(1, 1, 64, 100, 2, 4)
    assert need > 0
    _expect(_heads(ws_bytes=need - 1), WS, ["workspace"])
    _expect(_heads(ws=None), WS, ["workspace"])


def test_tree_build_candidates_errors():
    lib = _lib()
    _expect(lib.tree_build_candidates(None, -1, 4, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None), ARG, ["B < 0"])
    _expect(lib.tree_build_candidates(None, 2, 4, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None), ARG, ["null tree"])


def _attn(dtype=1, B=1, T=64, Hq=32, Hkv=8, Dh=128, Lmax=2048, L_hint=2048, ptrs=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return _lib().tree_attention(dtype, B, T, Hq, Hkv, Dh, ptrs, FAKE, FAKE, Lmax, L_hint, FAKE, FAKE, FAKE, FAKE,
                                 C.c_float(0.1), FAKE, ws, ws_bytes, None)


def test_tree_attention_errors():
    _expect(_attn(dtype=3), UNSUP, ["dtype"])
    _expect(_attn(Hq=30), ARG, ["not a multiple"])
    _expect(_attn(T=65), UNSUP, ["T=65"])
    _expect(_attn(T=0), ARG, ["bad sizes"])
    _expect(_attn(L_hint=4096), ARG, ["L_hint"])
    _expect(_attn(ptrs=None), ARG, ["null pointer"])
    need = _lib().tree_attention_workspace_size(1, 1, 64, 32, 8, 128, 2048)
    assert need > 0
    _expect(_attn(ws_bytes=need - 1), WS, ["workspace"])
    _expect(_attn(ws=None, ws_bytes=need), WS, ["workspace"])
    _expect(_attn(dtype=0, Dh=256, ws=None, ws_bytes=0), UNSUP, ["Dh <= 128"])


def test_tree_attention_noalloc_rejects_beyond_its_scratch():
    lib = _lib()
    cap = lib.tree_attention_noalloc_max_scratch()
    assert cap == 64 << 20
    # batch 51, 20/5 heads, prefix 65536: 64.7 MiB of split partials
    need = lib.tree_attention_workspace_size(1, 51, 64, 20, 5, 128, 65536)
    assert need > cap
    rc = lib.tree_attention_noalloc(1, 51, 64, 20, 5, 128, FAKE, FAKE, FAKE, 65536, 65536, FAKE, FAKE, FAKE, FAKE,
                                    C.c_float(0.1), FAKE, None)
    _expect(rc, WS, ["static scratch"])


def _post(B=2, V=100, mode=1, tau=0.7, tree=None, ws_bytes=1 << 20):
    return _lib().evaluate_posterior(tree, B, V, FAKE, FAKE, mode, C.c_float(tau), C.c_float(0.09),
                                     C.c_float(0.3), FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)


def test_evaluate_posterior_errors():
    _expect(_post(V=0), ARG, ["bad sizes"])
    _expect(_post(mode=5), ARG, ["mode 5"])
    _expect(_post(tau=0.0), ARG, ["temperature"])
    _expect(_post(), ARG, ["null tree"])


def _compact(dtype=1, NL=2, B=2, Hkv=8, Dh=128, Lmax=100, out_tokens=None, n_out=None, max_new=0):
    return _lib().kv_compact(dtype, None, NL, B, Hkv, Dh, Lmax, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             out_tokens, max_new, n_out, None, None)


def test_kv_compact_errors():
    _expect(_compact(dtype=9), UNSUP, ["dtype"])
    _expect(_compact(Lmax=0), ARG, ["bad sizes"])
    _expect(_compact(Hkv=0), ARG, ["bad sizes"])
    _expect(_compact(dtype=1, Dh=4), UNSUP, ["16 bytes"])
    _expect(_compact(out_tokens=FAKE, n_out=None, max_new=8), ARG, ["needs n_out"])
    _expect(_compact(), ARG, ["null tree"])


def test_sampling_calls_errors():
    from speculative_decoding_heads_amd._lib import SamplingDesc
    lib = _lib()
    good = SamplingDesc(1, 0.7, 0.09, 0.3, 0.8, 1)
    _expect(lib.medusa_sample_tokens(None, 4, 100, FAKE, 100, None, FAKE, FAKE, None), ARG, ["null parameters"])
    _expect(lib.medusa_sample_tokens(C.byref(SamplingDesc(3, 0.7, 0.09, 0.3, 0.8, 1)), 4, 100, FAKE, 100, None,
                                     FAKE, FAKE, None), ARG, ["kind 3"])
    _expect(lib.medusa_sample_tokens(C.byref(SamplingDesc(2, 0.0, 0.09, 0.3, 0.8, 1)), 4, 100, FAKE, 100, None,
                                     FAKE, FAKE, None), ARG, ["temperature"])
    _expect(lib.medusa_sample_tokens(C.byref(good), 4, 100, FAKE, 99, None, FAKE, FAKE, None), ARG, ["bad sizes"])
    _expect(lib.medusa_sample_tokens(C.byref(good), 4, 100, FAKE, 100, None, None, FAKE, None), ARG,
            ["null pointer"])
    _expect(lib.evaluate_posterior_sampled(None, 2, 100, FAKE, FAKE, FAKE, C.byref(good), FAKE, FAKE, FAKE, FAKE,
                                           FAKE, 1 << 20, None), ARG, ["null tree"])


def _forward_with(**over):
    """medusa_forward on a bf16 model description with fake device pointers: shape
    errors are reported before any device work."""
    from speculative_decoding_heads_amd._lib import LayerWeights, ModelDesc
    dims = dict(dtype=1, n_layers=1, d=512, n_heads=8, n_kv_heads=4, head_dim=64, ffn=1024, vocab=100)
    dims.update(over)
    layer = LayerWeights(*([FAKE.value] * 6))
    m = ModelDesc(dims["dtype"], dims["n_layers"], dims["d"], dims["n_heads"], dims["n_kv_heads"], dims["head_dim"],
                  dims["ffn"], dims["vocab"], 1e-6, FAKE.value, FAKE.value, FAKE.value, C.pointer(layer),
                  FAKE.value, FAKE.value, 256, 0, None, None)
    return _lib().medusa_forward(C.byref(m), 1, 8, FAKE, FAKE, FAKE, FAKE, 64, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, 1 << 30, None)


def test_forward_model_shape_errors():
    _expect(_forward_with(ffn=1000), UNSUP, ["multiples of 32", "ffn 1000"])
    _expect(_forward_with(d=520), UNSUP, ["multiples of 32", "d 520"])
    _expect(_forward_with(d=8224), UNSUP, ["d <= 8192"])
    _expect(_forward_with(n_heads=3, n_kv_heads=1, head_dim=48), UNSUP, ["multiples of 32"])
    _expect(_forward_with(head_dim=256, n_heads=2, n_kv_heads=2), UNSUP, ["head_dim 256 > 128"])
    _expect(_forward_with(n_heads=6, n_kv_heads=4), ARG, ["bad dimensions"])
