// The verify forward, prefill and one whole verify step, as stream-ordered
// sequences of the library's kernels (no host synchronisation, no allocation).
//
// medusa_step is one iteration of medusa_generate() on the page "大模型推理
// memory bandwidth bound (5) - Medusa" (section 二.1): generate_candidates
// (heads + top-K, tree expansion), tree_decoding (the base model over the T
// tree tokens with the tree mask), evaluate_posterior, update_inference_inputs
// (KV compaction, token append, the next root and the next heads' input taken
// at the node reached on the chosen path).
#include <vector>

#include "common.h"
#include "medusa_model.h"
#include "tree_dev.h"

using namespace medusa;

namespace {

__global__ void fill_i32_kernel(int32_t* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void add_i32_kernel(int32_t* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] += v;
}

__global__ void causal_anc_kernel(uint64_t* anc, int T) {
  const int i = threadIdx.x;
  if (i < T) anc[i] = (i == 63) ? ~0ull : ((1ull << (i + 1)) - 1ull);
}

// rows [b, t] of a chunk: tokens/pos from the prompt
__global__ void chunk_tokens_kernel(const int32_t* prompt, int S, int c0, int Sc, int32_t* tok, int32_t* pos) {
  const int b = blockIdx.x, t = threadIdx.x;
  if (t < Sc) {
    tok[b * Sc + t] = prompt[(size_t)b * S + c0 + t];
    pos[b * Sc + t] = c0 + t;
  }
}

// copy all T side-buffer rows of every (layer, b, h) to cache rows seq_len[b] + t
template <int EB>
__global__ void append_kv_kernel(int B, int Hkv, int T, int Dh, int64_t Lmax, char* Kc, char* Vc, const char* Kt,
                                 const char* Vt, const int32_t* seq_len) {
  const int lh = blockIdx.x, b = blockIdx.y;
  const int layer = lh / Hkv, h = lh % Hkv;
  const int s = seq_len[b];
  if (s < 0 || (int64_t)s + T > Lmax) return;
  char* dst = blockIdx.z == 0 ? Kc : Vc;
  const char* src = blockIdx.z == 0 ? Kt : Vt;
  const size_t row_bytes = (size_t)Dh * EB, chunks = row_bytes / 16;
  const size_t slab = ((size_t)layer * B + b) * Hkv + h;
  for (size_t e = threadIdx.x; e < (size_t)T * chunks; e += blockDim.x) {
    const size_t t = e / chunks, c = e % chunks;
    *((uint4*)(dst + (slab * Lmax + s + t) * row_bytes) + c) = *((const uint4*)(src + (slab * T + t) * row_bytes) + c);
  }
}

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += align_up(bytes, 256);
    return p;
  }
};

size_t gemm_ws_max(const medusa_model* m, int M) {
  const int d = m->d, Dh = m->head_dim, Hq = m->n_heads, Hkv = m->n_kv_heads, F = m->ffn, V = m->vocab;
  size_t w = 0;
  auto upd = [&](size_t x) { w = x > w ? x : w; };
  upd(medusa_gemm_workspace_size(m->dtype, M, (Hq + 2 * Hkv) * Dh, d, 1));
  upd(medusa_gemm_workspace_size(m->dtype, M, d, Hq * Dh, 1));
  upd(medusa_gemm_workspace_size(m->dtype, M, 2 * F, d, 1));
  upd(medusa_gemm_workspace_size(m->dtype, M, d, F, 1));
  upd(medusa_gemm_workspace_size(m->dtype, M, V, d, 1));
  upd(medusa_gemm_resid_rmsnorm_workspace_size(m->dtype, M, d, Hq * Dh));
  upd(medusa_gemm_resid_rmsnorm_workspace_size(m->dtype, M, d, F));
  return w;
}

struct FwdBufs {
  void *x, *xn, *qkv, *q, *attn, *act, *gws, *aws;
  size_t gws_bytes, aws_bytes;
};

size_t fwd_layout(const medusa_model* m, int B, int T, int64_t L_hint, void* ws, FwdBufs* fb) {
  const int M = B * T;
  const size_t es = dtype_size(m->dtype);
  const int Dh = m->head_dim, Hq = m->n_heads, Hkv = m->n_kv_heads;
  Carver c(ws);
  FwdBufs f;
  f.x = c.take((size_t)M * m->d * es);
  f.xn = c.take((size_t)M * m->d * es);
  f.qkv = c.take((size_t)M * (Hq + 2 * Hkv) * Dh * sizeof(float));
  f.q = c.take((size_t)M * Hq * Dh * es);
  f.attn = c.take((size_t)M * Hq * Dh * es);
  f.act = c.take((size_t)M * m->ffn * es);
  f.gws_bytes = gemm_ws_max(m, M);
  f.gws = c.take(f.gws_bytes);
  f.aws_bytes = tree_attention_workspace_size(m->dtype, B, T, Hq, Hkv, Dh, L_hint);
  f.aws = c.take(f.aws_bytes);
  if (fb) *fb = f;
  return c.off;
}

int check_model(const medusa_model* m) {
  MEDUSA_REQUIRE(m, MEDUSA_ERR_ARG, "model: null");
  MEDUSA_REQUIRE(dtype_ok(m->dtype), MEDUSA_ERR_UNSUPPORTED, "model: dtype %d", m->dtype);
  MEDUSA_REQUIRE(m->n_layers >= 1 && m->d > 0 && m->n_heads > 0 && m->n_kv_heads > 0 &&
                     m->n_heads % m->n_kv_heads == 0 && m->head_dim > 0 && m->head_dim % 2 == 0 && m->ffn > 0 &&
                     m->vocab > 0,
                 MEDUSA_ERR_ARG, "model: bad dimensions");
  // shapes every kernel of the forward takes, checked before anything is launched:
  // attention heads of at most 128; bf16 products step K by 32 (K = d, Hq * Dh and
  // ffn) and the residual norms hold a row of at most 8192
  MEDUSA_REQUIRE(m->head_dim <= 128, MEDUSA_ERR_UNSUPPORTED, "model: head_dim %d > 128", m->head_dim);
  MEDUSA_REQUIRE(m->dtype != MEDUSA_BF16 || (m->d % 32 == 0 && (m->n_heads * m->head_dim) % 32 == 0 &&
                                             m->ffn % 32 == 0 && m->d <= 8192),
                 MEDUSA_ERR_UNSUPPORTED,
                 "model: bf16 needs d, n_heads * head_dim and ffn multiples of 32 and d <= 8192 (d %d, %d, ffn %d)",
                 m->d, m->n_heads * m->head_dim, m->ffn);
  MEDUSA_REQUIRE(m->layers && m->embed && m->final_norm && m->lm_head && m->rope_cos && m->rope_sin &&
                     m->rope_max_pos > 0,
                 MEDUSA_ERR_ARG, "model: null weight pointer");
  return MEDUSA_OK;
}

}  // namespace

extern "C" size_t medusa_forward_workspace_size(const medusa_model* m, int B, int T, int64_t L_hint) {
  if (!m || B <= 0 || T <= 0) return 0;
  return fwd_layout(m, B, T, L_hint, nullptr, nullptr);
}

namespace {
int forward_impl(const medusa_model* m, int B, int T, const int32_t* tokens, const int32_t* pos, const void* Kc,
                 const void* Vc, int64_t Lmax, int64_t L_hint, const int32_t* seq_len, void* Kt, void* Vt,
                 const uint64_t* anc, float* logits, void* h, const medusa_trace* tr, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  int rc = check_model(m);
  if (rc) return rc;
  MEDUSA_REQUIRE(B >= 0 && T >= 1 && T <= MEDUSA_MAX_TREE, MEDUSA_ERR_ARG, "forward: bad B/T");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(tokens && pos && seq_len && Kt && Vt && anc && logits && h, MEDUSA_ERR_ARG, "forward: null pointer");
  FwdBufs f;
  const size_t need = fwd_layout(m, B, T, L_hint, ws, &f);
  MEDUSA_REQUIRE(ws && ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "forward: workspace %zu < %zu", ws_bytes, need);
  const int dt = m->dtype, M = B * T, d = m->d, Dh = m->head_dim, Hq = m->n_heads, Hkv = m->n_kv_heads, F = m->ffn;
  const size_t es = dtype_size(dt);
  const size_t cache_layer = (size_t)B * Hkv * Lmax * Dh * es;
  const size_t side_layer = (size_t)B * Hkv * T * Dh * es;
  const float scale = 1.0f / sqrtf((float)Dh);
#define CK(x)          \
  do {                 \
    int r_ = (x);      \
    if (r_) return r_; \
  } while (0)
  // tracing: copy a stage's output into slot `slot` of a caller buffer (skipped when null)
  auto trace = [&](void* dst, int slot, const void* src, size_t row_elems) -> int {
    if (!dst) return MEDUSA_OK;
    const size_t bytes = (size_t)M * row_elems * es;
    MEDUSA_HIP(hipMemcpyAsync((char*)dst + slot * bytes, src, bytes, hipMemcpyDeviceToDevice, stream));
    return MEDUSA_OK;
  };
  const medusa_trace none = {};
  const medusa_trace& t = tr ? *tr : none;
  // the embedding gather also applies the first layer's input RMSNorm, and each
  // residual projection the RMSNorm that feeds the next sub-layer (the last one
  // the final norm, into h)
  CK(embed_rmsnorm(dt, M, d, tokens, m->embed, m->vocab, m->layers[0].attn_norm, m->norm_eps, f.x, f.xn, stream));
  CK(trace(t.x, 0, f.x, d));
  for (int l = 0; l < m->n_layers; ++l) {
    const medusa_layer_weights& w = m->layers[l];
    const bool last = l + 1 == m->n_layers;
    char* kt = (char*)Kt + l * side_layer;
    char* vt = (char*)Vt + l * side_layer;
    CK(trace(t.xn, l, f.xn, d));
    // bf16: the product's epilogue applies the rotary embedding and splits q/K/V
    const int fused = dt == MEDUSA_BF16
                          ? gemm_qkv_rope_bf16(B, T, d, Hq, Hkv, Dh, (const bf16_t*)f.xn, (const bf16_t*)w.wqkv, pos,
                                               m->rope_cos, m->rope_sin, m->rope_max_pos, (bf16_t*)f.q, (bf16_t*)kt,
                                               (bf16_t*)vt, stream)
                          : MEDUSA_ERR_UNSUPPORTED;
    if (fused != MEDUSA_OK && fused != MEDUSA_ERR_UNSUPPORTED) return fused;
    if (fused == MEDUSA_ERR_UNSUPPORTED) {
      CK(medusa_gemm(dt, M, (Hq + 2 * Hkv) * Dh, d, f.xn, d, 0, w.wqkv, 0, f.qkv, (Hq + 2 * Hkv) * Dh, 0, 1,
                     MEDUSA_EPI_F32, nullptr, 0, 0, f.gws, f.gws_bytes, stream));
      CK(medusa_rope_split(dt, B, T, Hq, Hkv, Dh, (const float*)f.qkv, pos, m->rope_cos, m->rope_sin,
                           m->rope_max_pos, f.q, kt, vt, stream));
    }
    CK(trace(t.q, l, f.q, (size_t)Hq * Dh));
    CK(tree_attention(dt, B, T, Hq, Hkv, Dh, f.q, Lmax ? (const char*)Kc + l * cache_layer : nullptr,
                      Lmax ? (const char*)Vc + l * cache_layer : nullptr, Lmax, L_hint, seq_len, kt, vt, anc, scale,
                      f.attn, f.aws, f.aws_bytes, stream));
    CK(trace(t.attn, l, f.attn, (size_t)Hq * Dh));
    CK(medusa_gemm_resid_rmsnorm(dt, M, d, Hq * Dh, f.attn, Hq * Dh, w.wo, f.x, w.ffn_norm, m->norm_eps, f.xn, f.gws,
                                 f.gws_bytes, stream));
    CK(trace(t.x_mid, l, f.x, d));
    CK(medusa_gemm(dt, M, 2 * F, d, f.xn, d, 0, w.w_gate_up, 0, f.act, F, 0, 1, MEDUSA_EPI_SWIGLU, nullptr, 0, 0,
                   f.gws, f.gws_bytes, stream));
    CK(trace(t.act, l, f.act, F));
    CK(medusa_gemm_resid_rmsnorm(dt, M, d, F, f.act, F, w.w_down, f.x, last ? m->final_norm : m->layers[l + 1].attn_norm,
                                 m->norm_eps, last ? h : f.xn, f.gws, f.gws_bytes, stream));
    CK(trace(t.x, l + 1, f.x, d));
  }
  CK(medusa_gemm(dt, M, m->vocab, d, h, d, 0, m->lm_head, 0, logits, m->vocab, 0, 1, MEDUSA_EPI_F32, nullptr, 0, 0,
                 f.gws, f.gws_bytes, stream));
  return MEDUSA_OK;
}
}  // namespace

extern "C" int medusa_forward(const medusa_model* m, int B, int T, const int32_t* tokens, const int32_t* pos,
                              const void* Kc, const void* Vc, int64_t Lmax, int64_t L_hint, const int32_t* seq_len,
                              void* Kt, void* Vt, const uint64_t* anc, float* logits, void* h, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  return forward_impl(m, B, T, tokens, pos, Kc, Vc, Lmax, L_hint, seq_len, Kt, Vt, anc, logits, h, nullptr, ws,
                      ws_bytes, stream);
}

extern "C" int medusa_forward_trace(const medusa_model* m, int B, int T, const int32_t* tokens, const int32_t* pos,
                                    const void* Kc, const void* Vc, int64_t Lmax, int64_t L_hint,
                                    const int32_t* seq_len, void* Kt, void* Vt, const uint64_t* anc, float* logits,
                                    void* h, const medusa_trace* trace, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  MEDUSA_REQUIRE(trace, MEDUSA_ERR_ARG, "forward_trace: null trace");
  return forward_impl(m, B, T, tokens, pos, Kc, Vc, Lmax, L_hint, seq_len, Kt, Vt, anc, logits, h, trace, ws,
                      ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// prefill
// ---------------------------------------------------------------------------
namespace {
struct PrefillBufs {
  int32_t *tok, *pos;
  uint64_t* anc;
  void *Kt, *Vt, *h;
  float* logits;
  void* fws;
  size_t fws_bytes;
};
size_t prefill_layout(const medusa_model* m, int B, int S, int64_t Lmax, void* ws, PrefillBufs* pb) {
  const int T = S < MEDUSA_MAX_TREE ? S : MEDUSA_MAX_TREE;
  const size_t es = dtype_size(m->dtype);
  Carver c(ws);
  PrefillBufs p;
  p.tok = (int32_t*)c.take((size_t)B * T * 4);
  p.pos = (int32_t*)c.take((size_t)B * T * 4);
  p.anc = (uint64_t*)c.take(MEDUSA_MAX_TREE * 8);
  const size_t side = (size_t)m->n_layers * B * m->n_kv_heads * T * m->head_dim * es;
  p.Kt = c.take(side);
  p.Vt = c.take(side);
  p.h = c.take((size_t)B * T * m->d * es);
  p.logits = (float*)c.take((size_t)B * T * m->vocab * sizeof(float));
  p.fws_bytes = fwd_layout(m, B, T, Lmax, nullptr, nullptr);
  p.fws = c.take(p.fws_bytes);
  if (pb) *pb = p;
  return c.off;
}
}  // namespace

extern "C" size_t medusa_prefill_workspace_size(const medusa_model* m, int B, int S, int64_t Lmax) {
  if (!m || B <= 0 || S <= 0) return 0;
  return prefill_layout(m, B, S, Lmax, nullptr, nullptr);
}

extern "C" int medusa_prefill(const medusa_model* m, int B, int S, const int32_t* prompt, medusa_state* st, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  int rc = check_model(m);
  if (rc) return rc;
  MEDUSA_REQUIRE(st && prompt && B >= 1 && S >= 1, MEDUSA_ERR_ARG, "prefill: bad arguments");
  MEDUSA_REQUIRE(S <= st->Lmax, MEDUSA_ERR_ARG, "prefill: prompt longer than the cache");
  MEDUSA_REQUIRE(st->Kc && st->Vc && st->seq_len && st->root && st->h_sel, MEDUSA_ERR_ARG, "prefill: null state");
  MEDUSA_REQUIRE(((size_t)m->head_dim * dtype_size(m->dtype)) % 16 == 0, MEDUSA_ERR_UNSUPPORTED,
                 "prefill: K/V rows must be multiples of 16 bytes");
  PrefillBufs p;
  const size_t need = prefill_layout(m, B, S, st->Lmax, ws, &p);
  MEDUSA_REQUIRE(ws && ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "prefill: workspace %zu < %zu", ws_bytes, need);
  hipLaunchKernelGGL(fill_i32_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, st->seq_len, B, 0);
  if (st->n_out) hipLaunchKernelGGL(fill_i32_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, st->n_out, B, 0);
  if (st->err) hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, stream, st->err, 1, 0);
  if (st->done) hipLaunchKernelGGL(fill_i32_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, st->done, B, 0);
  CK(check_launch("prefill init"));
  for (int c0 = 0; c0 < S; c0 += MEDUSA_MAX_TREE) {
    const int Sc = (S - c0) < MEDUSA_MAX_TREE ? (S - c0) : MEDUSA_MAX_TREE;
    hipLaunchKernelGGL(causal_anc_kernel, dim3(1), dim3(64), 0, stream, p.anc, Sc);
    hipLaunchKernelGGL(chunk_tokens_kernel, dim3(B), dim3(64), 0, stream, prompt, S, c0, Sc, p.tok, p.pos);
    CK(check_launch("prefill chunk setup"));
    CK(medusa_forward(m, B, Sc, p.tok, p.pos, st->Kc, st->Vc, st->Lmax, c0, st->seq_len, p.Kt, p.Vt, p.anc, p.logits,
                      p.h, p.fws, p.fws_bytes, stream));
    dim3 g(m->n_layers * m->n_kv_heads, B, 2);
    if (m->dtype == MEDUSA_BF16)
      hipLaunchKernelGGL(append_kv_kernel<2>, g, dim3(128), 0, stream, B, m->n_kv_heads, Sc, m->head_dim, st->Lmax,
                         (char*)st->Kc, (char*)st->Vc, (const char*)p.Kt, (const char*)p.Vt, st->seq_len);
    else
      hipLaunchKernelGGL(append_kv_kernel<4>, g, dim3(128), 0, stream, B, m->n_kv_heads, Sc, m->head_dim, st->Lmax,
                         (char*)st->Kc, (char*)st->Vc, (const char*)p.Kt, (const char*)p.Vt, st->seq_len);
    hipLaunchKernelGGL(add_i32_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, st->seq_len, B, Sc);
    CK(check_launch("prefill append"));
    if (c0 + Sc == S) {
      if (st->sampling) {
        // the root drawn from the last prompt position's logits (position S - 1)
        hipLaunchKernelGGL(fill_i32_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, p.pos, B, S - 1);
        CK(check_launch("prefill root position"));
        CK(medusa_sample_tokens(st->sampling, B, m->vocab, p.logits + (size_t)(Sc - 1) * m->vocab,
                                (int64_t)Sc * m->vocab, nullptr, p.pos, st->root, stream));
      } else {
        CK(medusa_argmax_rows(B, m->vocab, p.logits + (size_t)(Sc - 1) * m->vocab, (int64_t)Sc * m->vocab,
                              st->root, stream));
      }
      // h_sel[b] = h[b, Sc-1]: gather with a constant selector
      int32_t* selbuf = p.tok;  // reuse: B entries
      hipLaunchKernelGGL(fill_i32_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, selbuf, B, Sc - 1);
      CK(check_launch("prefill select"));
      CK(medusa_gather_rows(m->dtype, B, Sc, m->d, p.h, selbuf, st->h_sel, stream));
    }
  }
  return MEDUSA_OK;
}

// ---------------------------------------------------------------------------
// one verify step
// ---------------------------------------------------------------------------
namespace {
struct StepBufs {
  int32_t *topk, *tok, *pos, *cart, *next_root, *appended;
  void *Kt, *Vt, *h;
  float* logits;
  void *hws, *fws, *pws;
  size_t hws_bytes, fws_bytes, pws_bytes;
};
size_t step_layout(const medusa_model* m, const medusa_tree* t, int B, int64_t L_hint, void* ws, StepBufs* sb) {
  const int T = t->host.T, P = t->host.P, D = t->host.D, K = t->host.K, H = m->n_medusa;
  const size_t es = dtype_size(m->dtype);
  Carver c(ws);
  StepBufs s;
  s.topk = (int32_t*)c.take((size_t)B * H * K * 4);
  s.tok = (int32_t*)c.take((size_t)B * T * 4);
  s.pos = (int32_t*)c.take((size_t)B * T * 4);
  s.cart = (int32_t*)c.take((size_t)B * P * (D + 1) * 4);
  s.next_root = (int32_t*)c.take((size_t)B * 4);
  s.appended = (int32_t*)c.take((size_t)B * 4);
  const size_t side = (size_t)m->n_layers * B * m->n_kv_heads * T * m->head_dim * es;
  s.Kt = c.take(side);
  s.Vt = c.take(side);
  s.h = c.take((size_t)B * T * m->d * es);
  s.logits = (float*)c.take((size_t)B * T * m->vocab * sizeof(float));
  s.hws_bytes = medusa_heads_topk_workspace_size(m->dtype, B, m->d, m->vocab, H, K);
  s.hws = c.take(s.hws_bytes);
  s.fws_bytes = fwd_layout(m, B, T, L_hint, nullptr, nullptr);
  s.fws = c.take(s.fws_bytes);
  s.pws_bytes = evaluate_posterior_workspace_size(B, T);
  if (evaluate_posterior_sampled_workspace_size(B, T) > s.pws_bytes)
    s.pws_bytes = evaluate_posterior_sampled_workspace_size(B, T);
  s.pws = c.take(s.pws_bytes);
  if (sb) *sb = s;
  return c.off;
}
}  // namespace

namespace {
// KV compaction and token append of a step, with per-sequence stop when the
// state carries done flags; appended[b] says whether sequence b took all its
// accepted tokens
int compact_state(const medusa_model* m, const medusa_tree* t, int B, medusa_state* st, const void* Kt,
                  const void* Vt, const int32_t* tok, int32_t* appended, hipStream_t stream) {
  if (st->done)
    return kv_compact_stop(m->dtype, t, m->n_layers, B, m->n_kv_heads, m->head_dim, st->Lmax, st->Kc, st->Vc, Kt, Vt,
                           st->best, st->accept_len, st->seq_len, tok, st->out_tokens, st->max_new, st->n_out,
                           st->done, st->stop_token, st->err, appended, stream);
  return kv_compact_flags(m->dtype, t, m->n_layers, B, m->n_kv_heads, m->head_dim, st->Lmax, st->Kc, st->Vc, Kt, Vt,
                          st->best, st->accept_len, st->seq_len, tok, st->out_tokens, st->max_new, st->n_out, st->err,
                          appended, stream);
}

// Acceptance of a step: the fast rule (greedy / typical) or, for MEDUSA_SAMPLED,
// the draw-matching non-fast branch; next_root goes to the step workspace.
int accept_step(const medusa_model* m, const medusa_tree* t, int B, int mode, float temperature, float eps,
                float delta, medusa_state* st, const StepBufs& s, hipStream_t stream) {
  if (mode == MEDUSA_SAMPLED) {
    MEDUSA_REQUIRE(st->sampling, MEDUSA_ERR_ARG, "step: mode MEDUSA_SAMPLED needs state sampling parameters");
    return evaluate_posterior_sampled(t, B, m->vocab, s.logits, s.tok, s.pos, st->sampling, st->best,
                                      st->accept_len, st->sel_node, s.next_root, s.pws, s.pws_bytes, stream);
  }
  return evaluate_posterior(t, B, m->vocab, s.logits, s.tok, mode, temperature, eps, delta, st->best,
                            st->accept_len, st->sel_node, s.next_root, s.pws, s.pws_bytes, stream);
}

// The next step's inputs, for the sequences that appended this step's tokens:
// root[b] = next_root[b] and h_sel[b] = h[b, sel[b]] (section 二.7: the next
// candidates come from the position the accepted path ends at).  A sequence
// that appended nothing (cache or output full, finished) keeps both, so its
// state still matches its cache.
template <typename TY>
__global__ void commit_step_kernel(int T, int d, const TY* __restrict__ h, const int32_t* __restrict__ sel,
                                   const int32_t* __restrict__ appended, const int32_t* __restrict__ next_root,
                                   int32_t* __restrict__ root, TY* __restrict__ h_sel) {
  const int b = blockIdx.x;
  if (!appended[b]) return;
  int s = sel[b];
  s = s < 0 ? 0 : (s >= T ? T - 1 : s);
  const TY* src = h + ((size_t)b * T + s) * d;
  TY* dst = h_sel + (size_t)b * d;
  // 16-byte pieces when the rows allow (d * sizeof(TY) % 16 == 0, aligned bases)
  constexpr int PE = 16 / sizeof(TY);
  if (d % PE == 0 && ((((uintptr_t)h) | ((uintptr_t)h_sel)) & 15) == 0) {
    for (int n = threadIdx.x; n < d / PE; n += blockDim.x) ((uint4*)dst)[n] = ((const uint4*)src)[n];
  } else {
    for (int n = threadIdx.x; n < d; n += blockDim.x) dst[n] = src[n];
  }
  if (threadIdx.x == 0) root[b] = next_root[b];
}

int commit_step(const medusa_model* m, int B, int T, const StepBufs& s, medusa_state* st, hipStream_t stream) {
  if (m->dtype == MEDUSA_BF16)
    hipLaunchKernelGGL(commit_step_kernel<bf16_t>, dim3(B), dim3(256), 0, stream, T, m->d, (const bf16_t*)s.h,
                       st->sel_node, s.appended, s.next_root, st->root, (bf16_t*)st->h_sel);
  else
    hipLaunchKernelGGL(commit_step_kernel<float>, dim3(B), dim3(256), 0, stream, T, m->d, (const float*)s.h,
                       st->sel_node, s.appended, s.next_root, st->root, (float*)st->h_sel);
  return check_launch("step commit");
}
}  // namespace

extern "C" size_t medusa_step_workspace_size(const medusa_model* m, const medusa_tree* t, int B, int64_t L_hint) {
  if (!m || !t || B <= 0 || m->n_medusa <= 0) return 0;
  return step_layout(m, t, B, L_hint, nullptr, nullptr);
}

extern "C" int medusa_step(const medusa_model* m, const medusa_tree* t, int B, int mode, float temperature, float eps,
                           float delta, medusa_state* st, int64_t L_hint, const int32_t* topk_override, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  int rc = check_model(m);
  if (rc) return rc;
  MEDUSA_REQUIRE(t && st && B >= 1, MEDUSA_ERR_ARG, "step: bad arguments");
  MEDUSA_REQUIRE(m->n_medusa >= t->host.D && m->medusa_w1 && m->medusa_w2, MEDUSA_ERR_ARG,
                 "step: the model has %d Medusa heads, the tree needs %d", m->n_medusa, t->host.D);
  MEDUSA_REQUIRE(L_hint >= 0 && L_hint <= st->Lmax, MEDUSA_ERR_ARG, "step: L_hint outside [0, Lmax]");
  MEDUSA_REQUIRE(st->best && st->accept_len && st->sel_node && st->h_sel && st->root && st->seq_len, MEDUSA_ERR_ARG,
                 "step: null state buffer");
  StepBufs s;
  const size_t need = step_layout(m, t, B, L_hint, ws, &s);
  MEDUSA_REQUIRE(ws && ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "step: workspace %zu < %zu", ws_bytes, need);
  const int H = m->n_medusa, K = t->host.K, T = t->host.T;
  const int32_t* topk = topk_override;
  if (!topk) {
    CK(medusa_heads_topk(m->dtype, B, m->d, m->vocab, H, K, st->h_sel, m->medusa_w1, m->medusa_w2, s.topk, nullptr,
                         s.hws, s.hws_bytes, stream));
    topk = s.topk;
  }
  CK(tree_build_candidates(t, B, H, K, st->root, topk, st->seq_len, s.tok, s.pos, s.cart, stream));
  CK(medusa_forward(m, B, T, s.tok, s.pos, st->Kc, st->Vc, st->Lmax, L_hint, st->seq_len, s.Kt, s.Vt, t->dev->anc,
                    s.logits, s.h, s.fws, s.fws_bytes, stream));
  CK(accept_step(m, t, B, mode, temperature, eps, delta, st, s, stream));
  CK(compact_state(m, t, B, st, s.Kt, s.Vt, s.tok, s.appended, stream));
  CK(commit_step(m, B, T, s, st, stream));
  return MEDUSA_OK;
#undef CK
}

// ---------------------------------------------------------------------------
// fused draft + verify: the heads on every tree node inside the step
// ---------------------------------------------------------------------------
namespace {

// carry[b] = all[b * T + sel[b]]: the H*K top-K entries of the node each
// sequence's accepted path ends at (sel clamped to [0, T)); kept unchanged for
// a sequence that appended nothing this step
__global__ void gather_topk_kernel(int T, int HK, const int32_t* __restrict__ all, const int32_t* __restrict__ sel,
                                   const int32_t* __restrict__ appended, int32_t* __restrict__ carry) {
  const int b = blockIdx.x;
  if (!appended[b]) return;
  int s = sel[b];
  s = s < 0 ? 0 : (s >= T ? T - 1 : s);
  for (int i = threadIdx.x; i < HK; i += blockDim.x) carry[(size_t)b * HK + i] = all[((size_t)b * T + s) * HK + i];
}

struct FusedBufs {
  int32_t* topk_all;
  void* hws;
  size_t hws_bytes;
  void* step_ws;
  size_t step_bytes;
};

size_t fused_layout(const medusa_model* m, const medusa_tree* t, int B, int64_t L_hint, void* ws, FusedBufs* fb) {
  const int T = t->host.T, K = t->host.K, H = m->n_medusa;
  Carver c(ws);
  FusedBufs f;
  f.topk_all = (int32_t*)c.take((size_t)B * T * H * K * 4);
  f.hws_bytes = medusa_heads_topk_workspace_size(m->dtype, B * T, m->d, m->vocab, H, K);
  f.hws = c.take(f.hws_bytes);
  f.step_bytes = step_layout(m, t, B, L_hint, nullptr, nullptr);
  f.step_ws = c.take(f.step_bytes);
  if (fb) *fb = f;
  return c.off;
}

}  // namespace

extern "C" size_t medusa_step_fused_workspace_size(const medusa_model* m, const medusa_tree* t, int B,
                                                   int64_t L_hint) {
  if (!m || !t || B <= 0 || m->n_medusa <= 0) return 0;
  return fused_layout(m, t, B, L_hint, nullptr, nullptr);
}

extern "C" int medusa_step_fused(const medusa_model* m, const medusa_tree* t, int B, int mode, float temperature,
                                 float eps, float delta, medusa_state* st, int32_t* topk_carry, int64_t L_hint,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_model(m);
  if (rc) return rc;
  MEDUSA_REQUIRE(t && st && B >= 1 && topk_carry, MEDUSA_ERR_ARG, "step_fused: bad arguments");
  MEDUSA_REQUIRE(m->n_medusa >= t->host.D && m->medusa_w1 && m->medusa_w2, MEDUSA_ERR_ARG,
                 "step_fused: the model has %d Medusa heads, the tree needs %d", m->n_medusa, t->host.D);
  MEDUSA_REQUIRE(L_hint >= 0 && L_hint <= st->Lmax, MEDUSA_ERR_ARG, "step_fused: L_hint outside [0, Lmax]");
  MEDUSA_REQUIRE(st->best && st->accept_len && st->sel_node && st->h_sel && st->root && st->seq_len, MEDUSA_ERR_ARG,
                 "step_fused: null state buffer");
  FusedBufs f;
  const size_t need = fused_layout(m, t, B, L_hint, ws, &f);
  MEDUSA_REQUIRE(ws && ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "step_fused: workspace %zu < %zu", ws_bytes, need);
  StepBufs s;
  step_layout(m, t, B, L_hint, f.step_ws, &s);
  const int H = m->n_medusa, K = t->host.K, T = t->host.T;
#define CK(x)          \
  do {                 \
    int r_ = (x);      \
    if (r_) return r_; \
  } while (0)
  // this step's candidates: the top-K the previous step kept at its selected node
  CK(tree_build_candidates(t, B, H, K, st->root, topk_carry, st->seq_len, s.tok, s.pos, s.cart, stream));
  CK(medusa_forward(m, B, T, s.tok, s.pos, st->Kc, st->Vc, st->Lmax, L_hint, st->seq_len, s.Kt, s.Vt, t->dev->anc,
                    s.logits, s.h, s.fws, s.fws_bytes, stream));
  // the heads on the final hidden state of every tree node (B*T rows)
  CK(medusa_heads_topk(m->dtype, B * T, m->d, m->vocab, H, K, s.h, m->medusa_w1, m->medusa_w2, f.topk_all, nullptr,
                       f.hws, f.hws_bytes, stream));
  CK(accept_step(m, t, B, mode, temperature, eps, delta, st, s, stream));
  CK(compact_state(m, t, B, st, s.Kt, s.Vt, s.tok, s.appended, stream));
  CK(commit_step(m, B, T, s, st, stream));
  hipLaunchKernelGGL(gather_topk_kernel, dim3(B), dim3(64), 0, stream, T, H * K, f.topk_all, st->sel_node,
                     s.appended, topk_carry);
  return check_launch("step_fused carry");
#undef CK
}

// ---------------------------------------------------------------------------
// the step as a HIP graph: one launch replays the ~400 kernels of a step
// ---------------------------------------------------------------------------
struct medusa_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

extern "C" int medusa_step_graph_create(const medusa_model* m, const medusa_tree* t, int B, int mode,
                                        float temperature, float eps, float delta, medusa_state* st, int64_t L_hint,
                                        const int32_t* topk_override, void* ws, size_t ws_bytes, hipStream_t stream,
                                        medusa_graph** out) {
  MEDUSA_REQUIRE(out, MEDUSA_ERR_ARG, "step_graph_create: out is null");
  *out = nullptr;
  MEDUSA_REQUIRE(stream != nullptr, MEDUSA_ERR_ARG, "step_graph_create: capture needs a non-default stream");
  MEDUSA_HIP(hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal));
  const int rc = medusa_step(m, t, B, mode, temperature, eps, delta, st, L_hint, topk_override, ws, ws_bytes, stream);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(stream, &g);
  if (rc) {
    if (e == hipSuccess && g) (void)hipGraphDestroy(g);
    return rc;
  }
  if (e != hipSuccess) return fail(MEDUSA_ERR_HIP, "step_graph_create: end capture: %s", hipGetErrorString(e));
  hipGraphExec_t ex = nullptr;
  const hipError_t e2 = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  if (e2 != hipSuccess) {
    (void)hipGraphDestroy(g);
    return fail(MEDUSA_ERR_HIP, "step_graph_create: instantiate: %s", hipGetErrorString(e2));
  }
  medusa_graph* mg = new medusa_graph{g, ex};
  *out = mg;
  return MEDUSA_OK;
}

extern "C" int medusa_graph_launch(medusa_graph* g, hipStream_t stream) {
  MEDUSA_REQUIRE(g, MEDUSA_ERR_ARG, "graph_launch: null graph");
  MEDUSA_HIP(hipGraphLaunch(g->exec, stream));
  return MEDUSA_OK;
}

extern "C" int medusa_graph_destroy(medusa_graph* g) {
  if (!g) return MEDUSA_OK;
  hipError_t e1 = hipGraphExecDestroy(g->exec);
  hipError_t e2 = hipGraphDestroy(g->graph);
  delete g;
  if (e1 != hipSuccess || e2 != hipSuccess) return fail(MEDUSA_ERR_HIP, "graph_destroy failed");
  return MEDUSA_OK;
}
