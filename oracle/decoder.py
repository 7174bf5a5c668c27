"""Decoder forward over a batch of new tokens (the verify forward), plain greedy decode.

The pages leave the base model's layer shape open (the Ascend port names an
"openPangu dense" model; the code walk-through on "大模型推理 memory bandwidth
bound (5) - Medusa", section 二.5 ``tree_decoding()``, only fixes that the T
tree tokens run through the model in one forward with positions ``depth +
sequence length``, under the tree mask, and that logits and Medusa inputs come
out for every node).  Reading taken: a pre-norm LLaMA-style block --
RMSNorm (eps 1e-6) -> Q/K/V projections -> rotary embedding (theta 10000,
rotate-half) -> attention (oracle.attention) -> output projection + residual ->
RMSNorm -> SwiGLU FFN ``down(silu(gate x) * up x)`` + residual; a final RMSNorm
whose output h feeds both the LM head and the Medusa heads; no biases.

With ``bf16=True`` values are rounded to bfloat16 at the storage points of the
product path: the residual stream, each normed activation, q and k after the
rotary embedding, v, the attention output, the SwiGLU product, and h.  Logits
stay unrounded.

Weights are [out, in] matrices: y = x @ W.T.

Test infrastructure only (see ``oracle/__init__``).
"""
import numpy as np

from .attention import tree_attention
from .numerics import round_bf16, silu, argmax_first


def rmsnorm(x, w, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def rope(x, pos, theta=10000.0):
    """Rotate-half rotary embedding of x [..., Dh] at integer positions pos (broadcast over heads).

    x has shape [B, T, H, Dh] and pos [B, T]."""
    x = np.asarray(x, dtype=np.float64)
    Dh = x.shape[-1]
    half = Dh // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / Dh)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv  # [B, T, half]
    c = np.cos(ang)[:, :, None, :]
    s = np.sin(ang)[:, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _mm(x, W, mm_dtype):
    return (np.asarray(x, mm_dtype) @ np.asarray(W, mm_dtype).T).astype(np.float64)


def qkv_rotary(params, p, xn, pos, bf16=False, mm_dtype=np.float64):
    """Projections of the attention-normed rows xn [B, T, d] and the rotary embedding:
    (q [B, T, Hq, Dh], K [B, Hkv, T, Dh], V [B, Hkv, T, Dh])."""
    rb = round_bf16 if bf16 else (lambda v: v)
    Hq, Hkv, Dh = params["n_heads"], params["n_kv_heads"], params["head_dim"]
    B, T = xn.shape[:2]
    q = _mm(xn, p["wq"], mm_dtype).reshape(B, T, Hq, Dh)
    k = _mm(xn, p["wk"], mm_dtype).reshape(B, T, Hkv, Dh)
    v = _mm(xn, p["wv"], mm_dtype).reshape(B, T, Hkv, Dh)
    q = rb(rope(q, pos, params["rope_theta"]))
    k = rb(rope(k, pos, params["rope_theta"]))
    v = rb(v)
    return q, k.transpose(0, 2, 1, 3), v.transpose(0, 2, 1, 3)


def attention_residual(p, x, att, bf16=False, mm_dtype=np.float64):
    """Residual stream after the attention block: x + att W_o (att [B, T, Hq*Dh])."""
    rb = round_bf16 if bf16 else (lambda v: v)
    B, T = x.shape[:2]
    return rb(np.asarray(x, np.float64) + _mm(np.asarray(att).reshape(B, T, -1), p["wo"], mm_dtype))


def ffn_act(params, p, x_mid, bf16=False, mm_dtype=np.float64):
    """SwiGLU product of the FFN sub-layer: SiLU(gate) * up of the RMS-normed stream x_mid."""
    rb = round_bf16 if bf16 else (lambda v: v)
    xn2 = rb(rmsnorm(x_mid, p["ffn_norm"], params["norm_eps"]))
    return rb(silu(_mm(xn2, p["w_gate"], mm_dtype)) * _mm(xn2, p["w_up"], mm_dtype))


def down_residual(p, x_mid, act, bf16=False, mm_dtype=np.float64):
    """Residual stream leaving the layer: x_mid + act W_down."""
    rb = round_bf16 if bf16 else (lambda v: v)
    return rb(np.asarray(x_mid, np.float64) + _mm(act, p["w_down"], mm_dtype))


def decoder_layer(params, p, x, pos, cacheK, cacheV, seq_len, anc, bf16=False, mm_dtype=np.float64):
    """One pre-norm block over the new tokens' residual stream.

    p: the layer's weights; x [B, T, d] the residual stream entering the layer;
    pos [B, T]; cacheK, cacheV [B, Hkv, Lmax, Dh] this layer's cache with
    seq_len[b] valid rows; anc [T, T] bool visibility among the new tokens.
    Returns (x leaving the layer [B, T, d], K, V of the new tokens [B, Hkv, T, Dh]).
    """
    rb = round_bf16 if bf16 else (lambda v: v)
    x = np.asarray(x, np.float64)
    xn = rb(rmsnorm(x, p["attn_norm"], params["norm_eps"]))
    q, Kt, Vt = qkv_rotary(params, p, xn, pos, bf16, mm_dtype)
    att = rb(tree_attention(q, cacheK, cacheV, seq_len, Kt, Vt, anc, 1.0 / np.sqrt(params["head_dim"])))
    x = attention_residual(p, x, att, bf16, mm_dtype)
    x = down_residual(p, x, ffn_act(params, p, x, bf16, mm_dtype), bf16, mm_dtype)
    return x, Kt, Vt


def final_logits(params, x, bf16=False, mm_dtype=np.float64):
    """Final RMSNorm of the residual stream x [B, T, d] and the LM head: (logits, h)."""
    rb = round_bf16 if bf16 else (lambda v: v)
    h = rb(rmsnorm(x, params["final_norm"], params["norm_eps"]))
    return _mm(h, params["lm_head"], mm_dtype), h


def embed_tokens(params, tokens, bf16=False):
    """Residual stream entering the first layer: the embedding rows of the tokens [B, T]."""
    rb = round_bf16 if bf16 else (lambda v: v)
    return rb(np.asarray(params["embed"], np.float64)[np.asarray(tokens, dtype=np.int64)])


def forward(params, tokens, pos, cacheK, cacheV, seq_len, anc, bf16=False, mm_dtype=np.float64,
            layers=None):
    """Run the decoder over new tokens.

    tokens, pos [B, T];  cacheK, cacheV [NL, B, Hkv, Lmax, Dh] with seq_len[b] valid rows;
    anc [T, T] bool visibility among the new tokens.
    Returns (logits [B, T, V], h [B, T, d], Knew, Vnew [NL, B, Hkv, T, Dh]).
    ``layers`` limits the run to the first n layers (sampled checks); logits are
    then those of the truncated stack.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    B, T = tokens.shape
    Hkv, Dh = params["n_kv_heads"], params["head_dim"]
    x = embed_tokens(params, tokens, bf16)
    NL = len(params["layers"]) if layers is None else layers
    Knew = np.zeros((NL, B, Hkv, T, Dh))
    Vnew = np.zeros((NL, B, Hkv, T, Dh))
    for li in range(NL):
        x, Knew[li], Vnew[li] = decoder_layer(params, params["layers"][li], x, pos, cacheK[li], cacheV[li],
                                              seq_len, anc, bf16, mm_dtype)
    logits, h = final_logits(params, x, bf16, mm_dtype)
    return logits, h, Knew, Vnew


def empty_cache(params, B, Lmax):
    NL = len(params["layers"])
    shape = (NL, B, params["n_kv_heads"], Lmax, params["head_dim"])
    return np.zeros(shape), np.zeros(shape)


def write_cache(cacheK, cacheV, Knew, Vnew, seq_len):
    """Store new rows (all T of them, in order) right after each sequence's end."""
    T = Knew.shape[3]
    for b in range(cacheK.shape[1]):
        s = int(seq_len[b])
        cacheK[:, b, :, s:s + T] = Knew[:, b]
        cacheV[:, b, :, s:s + T] = Vnew[:, b]


def prefill(params, prompt, Lmax, bf16=False):
    """Causal forward over the prompt [B, S]; returns (logits, h, cacheK, cacheV, seq_len)."""
    prompt = np.asarray(prompt, dtype=np.int64)
    B, S = prompt.shape
    cK, cV = empty_cache(params, B, Lmax)
    seq = np.zeros(B, dtype=np.int64)
    pos = np.broadcast_to(np.arange(S), (B, S))
    anc = np.tril(np.ones((S, S), dtype=bool))
    logits, h, Kn, Vn = forward(params, prompt, pos, cK, cV, seq, anc, bf16=bf16)
    write_cache(cK, cV, Kn, Vn, seq)
    return logits, h, cK, cV, seq + S


def greedy_decode(params, prompt, n_new, Lmax, bf16=False):
    """Plain autoregressive greedy decoding: one token per forward.  Returns [B, n_new]."""
    logits, h, cK, cV, seq = prefill(params, prompt, Lmax, bf16=bf16)
    B = seq.shape[0]
    tok = argmax_first(logits[:, -1], axis=-1)
    out = [tok]
    one = np.ones((1, 1), dtype=bool)
    for _ in range(n_new - 1):
        logits, h, Kn, Vn = forward(params, tok[:, None], seq[:, None], cK, cV, seq, one, bf16=bf16)
        write_cache(cK, cV, Kn, Vn, seq)
        seq = seq + 1
        tok = argmax_first(logits[:, -1], axis=-1)
        out.append(tok)
    return np.stack(out, axis=1)
