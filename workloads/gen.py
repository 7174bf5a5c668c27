"""Seeded tensor generators (NumPy PCG64 on the host, or torch's generator on a device).

All draws are N(mean 0, std) or uniform integers, optionally rounded to
bfloat16 (nearest-even) so that the host copy and the device copy hold exactly
the same values.  Sizes follow the workloads: a tiny fp32 decoder, the Medusa
heads of a 4096-wide model with a 32000-token vocabulary, tree-attention inputs
of 32 query / 8 KV heads of width 128, and a 7B-shaped decoder.
"""
import numpy as np

__all__ = ["bf16_round", "bf16_bits", "normal", "TinyConfig", "SevenBConfig", "tiny_model",
           "heads_weights", "attention_inputs", "prompt_tokens", "torch_normal", "model_weights_torch"]


def bf16_round(x):
    """float32 array of the nearest bfloat16 values (ties to even)."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32)


def bf16_bits(x):
    """uint16 bit patterns of bf16-representable float32 values (truncation is exact for them)."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def normal(rng, shape, std=1.0, bf16=False):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_round(x) if bf16 else x


class TinyConfig:
    """Tiny fp32 Medusa step: 2-layer decoder, d 64, 4 heads x 16, SwiGLU 128, V 512, 2 heads."""
    n_layers = 2
    d = 64
    n_heads = 4
    n_kv_heads = 4
    head_dim = 16
    ffn = 128
    vocab = 512
    n_medusa = 2
    rope_theta = 10000.0
    norm_eps = 1e-6
    prompt_len = 32
    n_steps = 16


class SevenBConfig:
    """7B-shaped decoder: 32 layers, d 4096, 32 MHA heads x 128, SwiGLU 11008, V 32000, 4 heads."""
    n_layers = 32
    d = 4096
    n_heads = 32
    n_kv_heads = 32
    head_dim = 128
    ffn = 11008
    vocab = 32000
    n_medusa = 4
    rope_theta = 10000.0
    norm_eps = 1e-6


def tiny_model(seed=0, cfg=TinyConfig, std=0.02, bf16=False, n_layers=None):
    """Decoder parameters (float32 NumPy) and Medusa heads, all matrices N(0, std), norms 1."""
    rng = np.random.default_rng(seed)
    d, Hq, Hkv, Dh, F, V = cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.vocab
    NL = cfg.n_layers if n_layers is None else n_layers
    layers = []
    for _ in range(NL):
        layers.append(dict(
            attn_norm=np.ones(d, np.float32),
            wq=normal(rng, (Hq * Dh, d), std, bf16), wk=normal(rng, (Hkv * Dh, d), std, bf16),
            wv=normal(rng, (Hkv * Dh, d), std, bf16), wo=normal(rng, (d, Hq * Dh), std, bf16),
            ffn_norm=np.ones(d, np.float32),
            w_gate=normal(rng, (F, d), std, bf16), w_up=normal(rng, (F, d), std, bf16),
            w_down=normal(rng, (d, F), std, bf16)))
    params = dict(embed=normal(rng, (V, d), std, bf16), layers=layers,
                  final_norm=np.ones(d, np.float32), lm_head=normal(rng, (V, d), std, bf16),
                  n_heads=Hq, n_kv_heads=Hkv, head_dim=Dh, norm_eps=cfg.norm_eps,
                  rope_theta=cfg.rope_theta)
    heads = dict(W1=normal(rng, (cfg.n_medusa, d, d), std, bf16),
                 W2=normal(rng, (cfg.n_medusa, V, d), std, bf16))
    return params, heads


def heads_weights(seed=0, H=4, d=4096, V=32000, std=0.02, B=1, bf16=True):
    """(h [B, d] ~ N(0,1), W1 [H, d, d], W2 [H, V, d] ~ N(0, std)) as float32 (bf16 values)."""
    rng = np.random.default_rng(seed)
    h = normal(rng, (B, d), 1.0, bf16)
    W1 = normal(rng, (H, d, d), std, bf16)
    W2 = normal(rng, (H, V, d), std, bf16)
    return h, W1, W2


def attention_inputs(seed=0, B=1, T=64, Hq=32, Hkv=8, Dh=128, L=1024, Lmax=None, bf16=True,
                     ragged=False):
    """q [B,T,Hq,Dh], Kc/Vc [B,Hkv,Lmax,Dh], Kt/Vt [B,Hkv,T,Dh] ~ N(0,1), seq_len [B].

    With ``ragged`` the prefix lengths are drawn uniformly in [1, L]; otherwise all are L.
    Rows of the cache beyond seq_len are filled with NaN so that a read of them shows."""
    rng = np.random.default_rng(seed)
    Lmax = L if Lmax is None else Lmax
    q = normal(rng, (B, T, Hq, Dh), 1.0, bf16)
    Kc = normal(rng, (B, Hkv, Lmax, Dh), 1.0, bf16)
    Vc = normal(rng, (B, Hkv, Lmax, Dh), 1.0, bf16)
    Kt = normal(rng, (B, Hkv, T, Dh), 1.0, bf16)
    Vt = normal(rng, (B, Hkv, T, Dh), 1.0, bf16)
    if ragged:
        seq_len = rng.integers(1, L + 1, size=B).astype(np.int32)
    else:
        seq_len = np.full(B, L, dtype=np.int32)
    for b in range(B):
        Kc[b, :, seq_len[b]:] = np.nan
        Vc[b, :, seq_len[b]:] = np.nan
    return q, Kc, Vc, Kt, Vt, seq_len


def prompt_tokens(seed, B, S, V):
    rng = np.random.default_rng(seed)
    return rng.integers(0, V, size=(B, S)).astype(np.int64)


def torch_normal(shape, std, seed, device, dtype):
    """Seeded N(0, std) tensor drawn by torch's generator on ``device``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.empty(shape, device=device, dtype=torch.float32)
    t.normal_(0.0, std, generator=g)
    return t.to(dtype)


def model_weights_torch(cfg, seed, device, dtype, n_layers=None, std=0.02):
    """Decoder + Medusa head weights of ``cfg`` as torch tensors on ``device``.

    Each matrix gets its own seed (seed * 1000 + counter) so any subset can be
    regenerated alone; norm weights are 1."""
    import torch
    d, Hq, Hkv, Dh, F, V = cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.vocab
    NL = cfg.n_layers if n_layers is None else n_layers
    ctr = [seed * 1000]

    def mat(shape):
        ctr[0] += 1
        return torch_normal(shape, std, ctr[0], device, dtype)

    layers = []
    for _ in range(NL):
        layers.append(dict(
            attn_norm=torch.ones(d, device=device, dtype=dtype),
            wq=mat((Hq * Dh, d)), wk=mat((Hkv * Dh, d)), wv=mat((Hkv * Dh, d)), wo=mat((d, Hq * Dh)),
            ffn_norm=torch.ones(d, device=device, dtype=dtype),
            w_gate=mat((F, d)), w_up=mat((F, d)), w_down=mat((d, F))))
    params = dict(embed=mat((V, d)), layers=layers, final_norm=torch.ones(d, device=device, dtype=dtype),
                  lm_head=mat((V, d)), n_heads=Hq, n_kv_heads=Hkv, head_dim=Dh,
                  norm_eps=cfg.norm_eps, rope_theta=cfg.rope_theta)
    heads = dict(W1=mat((cfg.n_medusa, d, d)), W2=mat((cfg.n_medusa, V, d)))
    return params, heads
