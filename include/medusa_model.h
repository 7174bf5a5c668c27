/*
 * medusa_model.h -- building blocks of the verify forward (the base model run
 * over the T tree tokens, page "大模型推理 memory bandwidth bound (5) - Medusa",
 * section 二.5 tree_decoding) and the whole verify step.
 *
 * The pages leave the base model's layer shape open; the layer assumed here is
 * a pre-norm LLaMA-style block: RMSNorm -> fused Q/K/V projection -> rotary
 * embedding (rotate-half) -> tree attention -> output projection + residual ->
 * RMSNorm -> SwiGLU FFN + residual; a final RMSNorm feeds the LM head and the
 * Medusa heads.  Same conventions as medusa.h (status codes, caller-owned
 * device buffers, stream-ordered, no synchronisation, no allocation).
 */
#ifndef MEDUSA_MODEL_H
#define MEDUSA_MODEL_H

#include "medusa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Epilogues of medusa_gemm (acc = sum_k A[m,k] W[n,k] in fp32). */
enum {
  MEDUSA_EPI_F32 = 0,          /* C (fp32)[m,n] = acc                                  */
  MEDUSA_EPI_STORE = 1,        /* C (dtype)[m,n] = acc                                 */
  MEDUSA_EPI_RESID = 2,        /* C (dtype)[m,n] = R[m,n] + acc (R may alias C)        */
  MEDUSA_EPI_SILU_RESID_A = 3, /* C (dtype)[m,n] = A[m, n mod K] + SiLU(acc)  (Medusa
                                  head residual block, W1 stacked [H*K, K])             */
  MEDUSA_EPI_SWIGLU = 4        /* W rows interleaved gate/up: C (dtype)[m,j] =
                                  SiLU(acc[m,2j]) * acc[m,2j+1], j < N/2                 */
};

/*
 * Batched product: for z in [0, batch):  C_z = epi(A_z W_z^T)
 *   A_z = A + z*strideA, rows of length K with leading dimension lda (elements)
 *   W_z = W + z*strideW, [N, K] row-major
 *   C_z = C + z*strideC, leading dimension ldc;  R_z = R + z*strideR, ldr
 * bf16 needs K % 32 == 0 and 16-byte aligned rows; fp32 has no constraint.
 * Workspace (bf16 split-K partials) from medusa_gemm_workspace_size.
 */
size_t medusa_gemm_workspace_size(int dtype, int M, int N, int K, int batch);
int medusa_gemm(int dtype, int M, int N, int K, const void* A, int64_t lda, int64_t strideA, const void* W,
                int64_t strideW, void* C, int64_t ldc, int64_t strideC, int batch, int epilogue, const void* R,
                int64_t ldr, int64_t strideR, void* ws, size_t ws_bytes, hipStream_t stream);

/* y[m,:] = x[m,:] / sqrt(mean(x[m,:]^2) + eps) * w  (x, w, y in dtype; fp32 math) */
int medusa_rmsnorm(int dtype, int M, int N, const void* x, const void* w, float eps, void* y, hipStream_t stream);

/*
 * Residual projection followed by the next pre-norm (the decoder block's
 * "h = h + attn(.) W_o" / "h = h + mlp(.) W_down" and the RMSNorm that feeds the
 * next sub-layer), in one call:
 *   X[m,:] = X[m,:] + A[m,:] W^T        X [M, N] in dtype, updated in place
 *   Y[m,:] = X[m,:] / sqrt(mean(X[m,:]^2) + eps) * norm_w      (over the stored X)
 * A [M, K] with leading dimension lda, W [N, K].  bf16 needs K % 32 == 0,
 * N % 8 == 0, N <= 8192 and 16-byte aligned rows; the product's fp32 partials
 * go to the workspace and one kernel adds them, stores X and normalises.
 * fp32 runs the plain product and RMSNorm kernels.
 */
size_t medusa_gemm_resid_rmsnorm_workspace_size(int dtype, int M, int N, int K);
int medusa_gemm_resid_rmsnorm(int dtype, int M, int N, int K, const void* A, int64_t lda, const void* W, void* X,
                              const void* norm_w, float eps, void* Y, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Split a fused fp32 Q/K/V projection [B*T, (Hq + 2*Hkv)*Dh] into
 *   q  [B, T, Hq, Dh] (dtype) rotated at pos,   Kt [B, Hkv, T, Dh] rotated,   Vt [B, Hkv, T, Dh]
 * Rotary embedding, rotate-half: x'[i] = x[i] cos - x[i+Dh/2] sin, x'[i+Dh/2] = x[i+Dh/2] cos + x[i] sin,
 * angles from tables cos_tab/sin_tab [max_pos, Dh/2] (fp32, device).  Positions outside
 * [0, max_pos) are clamped.
 */
int medusa_rope_split(int dtype, int B, int T, int Hq, int Hkv, int Dh, const float* qkv, const int32_t* pos,
                      const float* cos_tab, const float* sin_tab, int max_pos, void* q_out, void* Kt, void* Vt,
                      hipStream_t stream);

/* out[m,:] = table[tokens[m], :]  (tokens clamped to [0, V)) */
int medusa_embed(int dtype, int M, int d, const int32_t* tokens, const void* table, int V, void* out,
                 hipStream_t stream);

/* out[b,:] = h[b, sel[b], :] for h [B, T, d] */
int medusa_gather_rows(int dtype, int B, int T, int d, const void* h, const int32_t* sel, void* out,
                       hipStream_t stream);

/* out[m] = argmax_v x[m*ldx + v] (lowest index on ties) for fp32 rows */
int medusa_argmax_rows(int M, int V, const float* x, int64_t ldx, int32_t* out, hipStream_t stream);

/* Top-K of fp32 rows: idx/val [M, K] (val nullable), value-descending, ties -> lower index; K <= 16 */
size_t medusa_topk_rows_workspace_size(int M, int V, int K);
int medusa_topk_rows(int M, int V, const float* x, int K, int32_t* idx, float* val, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * Streaming-read ceiling: n_workgroups workgroups each read a contiguous share
 * of src [bytes] (device, 16-byte aligned, bytes % 16 == 0) with 16-byte loads
 * and write one word to sink[n_workgroups] (device).  Measures the practical
 * HBM read rate that the memory-bound kernels are compared with (the page's
 * roofline remark, section 三, sets their bound by bytes moved).
 */
int medusa_read_probe(const void* src, size_t bytes, int n_workgroups, uint32_t* sink, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Whole model                                                                 */
/* ------------------------------------------------------------------------- */
typedef struct medusa_layer_weights {
  const void* attn_norm; /* [d]                                              */
  const void* wqkv;      /* [(Hq + 2 Hkv) Dh, d]: rows of Wq, then Wk, then Wv */
  const void* wo;        /* [d, Hq Dh]                                       */
  const void* ffn_norm;  /* [d]                                              */
  const void* w_gate_up; /* [2 F, d]: row 2j = gate j, row 2j+1 = up j       */
  const void* w_down;    /* [d, F]                                           */
} medusa_layer_weights;

typedef struct medusa_model {
  int dtype;
  int n_layers, d, n_heads, n_kv_heads, head_dim, ffn, vocab;
  float norm_eps;
  const void* embed;      /* [V, d]  */
  const void* final_norm; /* [d]     */
  const void* lm_head;    /* [V, d]  */
  const medusa_layer_weights* layers; /* HOST array of n_layers entries (device pointers inside) */
  const float* rope_cos;  /* [rope_max_pos, head_dim/2] device */
  const float* rope_sin;
  int rope_max_pos;
  /* Medusa heads */
  int n_medusa;
  const void* medusa_w1;  /* [H, d, d] */
  const void* medusa_w2;  /* [H, V, d] */
} medusa_model;

/*
 * Forward of B sequences x T new tokens (tokens, pos [B, T]) over the cache
 * Kc/Vc [n_layers, B, Hkv, Lmax, Dh] (seq_len valid rows) with visibility anc
 * (uint64 [T], device) among the new tokens.  Writes the new tokens' K/V to
 * Kt/Vt [n_layers, B, Hkv, T, Dh], logits [B, T, V] (fp32) and the final-normed
 * hidden state h [B, T, d] (dtype).  L_hint as in tree_attention.
 * Model shapes (checked first by every call that takes a model, which then
 * returns MEDUSA_ERR_UNSUPPORTED with nothing launched): head_dim <= 128; bf16
 * also needs d, n_heads * head_dim and ffn multiples of 32 and d <= 8192.
 */
size_t medusa_forward_workspace_size(const medusa_model* m, int B, int T, int64_t L_hint);
int medusa_forward(const medusa_model* m, int B, int T, const int32_t* tokens, const int32_t* pos, const void* Kc,
                   const void* Vc, int64_t Lmax, int64_t L_hint, const int32_t* seq_len, void* Kt, void* Vt,
                   const uint64_t* anc, float* logits, void* h, void* ws, size_t ws_bytes, hipStream_t stream);
/*
 * medusa_forward that also copies each stage's output into caller buffers, for
 * stage-by-stage checks against a reference (every pointer nullable, device,
 * caller-owned, in the model's dtype; rows are the B*T new tokens, b-major):
 *   x     [n_layers + 1, B*T, d]   residual stream entering layer l (slot 0: the
 *                                  embedding rows); slot n_layers: leaving the last
 *   xn    [n_layers, B*T, d]       the attention RMSNorm's output of layer l
 *   q     [n_layers, B*T, Hq*Dh]   rotated queries ([B, T, Hq, Dh] per layer)
 *   attn  [n_layers, B*T, Hq*Dh]   tree-attention output
 *   x_mid [n_layers, B*T, d]       residual stream after the attention block
 *   act   [n_layers, B*T, F]       SwiGLU product feeding the down projection
 * Same kernels and results as medusa_forward, plus one device copy per buffer
 * and layer.
 */
typedef struct medusa_trace {
  void* x;
  void* xn;
  void* q;
  void* attn;
  void* x_mid;
  void* act;
} medusa_trace;
int medusa_forward_trace(const medusa_model* m, int B, int T, const int32_t* tokens, const int32_t* pos,
                         const void* Kc, const void* Vc, int64_t Lmax, int64_t L_hint, const int32_t* seq_len,
                         void* Kt, void* Vt, const uint64_t* anc, float* logits, void* h, const medusa_trace* trace,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Generation state of B sequences (all device buffers, caller-owned):
 *   Kc, Vc [n_layers, B, Hkv, Lmax, Dh]; seq_len [B]; root [B] (next root token);
 *   h_sel [B, d] (Medusa-head input); out_tokens [B, max_new]; n_out [B]; err [1].
 * Step scratch (side buffers, logits, candidates) lives in the workspace.
 */
typedef struct medusa_state {
  void* Kc;
  void* Vc;
  int64_t Lmax;
  int32_t* seq_len;
  int32_t* root;
  void* h_sel;
  int32_t* out_tokens;
  int max_new;
  int32_t* n_out;
  int32_t* err;
  /* per-step outputs kept for inspection [B] each */
  int32_t* best;
  int32_t* accept_len;
  int32_t* sel_node;
  /* Per-sequence stop (nullable; the page's generation loop ends at the end-of-
   * sequence token, section 二.1).  With done [B] set, a step appends each
   * sequence's accepted tokens up to and including the first stop_token (< 0:
   * none) and within its output room (max_new - n_out) and cache room
   * (Lmax - seq_len); done[b] becomes 1 when it appends the stop token or fills
   * a room, and a sequence with done[b] = 1 appends nothing and keeps its cache
   * and length.  Prefill resets done to 0.  With done null, a step appends all
   * a+1 tokens and a full output or cache sets err instead. */
  int32_t* done;
  int32_t stop_token;
  /* Sampled generation (nullable, host pointer read at each call): prefill
   * draws the root at the last prompt position instead of taking the argmax,
   * and a step with mode MEDUSA_SAMPLED accepts by evaluate_posterior_sampled
   * (the non-fast branch) and takes the draw at the selected node as the next
   * root.  Null keeps the argmax root. */
  const medusa_sampling* sampling;
} medusa_state;

/*
 * Prefill: forward the prompt [B, S] (S <= 64 per chunk; longer prompts are
 * processed in chunks of 64 with a causal mask), write its K/V to the cache,
 * set seq_len = S, root = argmax of the last position's logits, h_sel = the
 * last position's final hidden state.  n_out is reset to 0.
 */
size_t medusa_prefill_workspace_size(const medusa_model* m, int B, int S, int64_t Lmax);
int medusa_prefill(const medusa_model* m, int B, int S, const int32_t* prompt, medusa_state* st, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/*
 * One verify iteration for B sequences sharing tree t (mode MEDUSA_GREEDY,
 * MEDUSA_TYPICAL -- the fast branch, temperature/eps/delta used -- or
 * MEDUSA_SAMPLED, which needs st->sampling and ignores temperature/eps/delta):
 *   Medusa heads + top-K on h_sel -> candidates -> forward of the T tree tokens
 *   -> acceptance -> KV compaction + token append -> h_sel, root for the next step.
 * best, accept_len and sel_node are written for every sequence; root and h_sel
 * change only for a sequence that appended all its accepted tokens, so one whose
 * cache or output was full (err set) or that is finished keeps the state its
 * cache and length describe.
 * L_hint: host upper bound of the sequence lengths during this step (<= Lmax).
 * topk_override [B, H, K] (nullable): when non-null, used instead of the heads'
 * top-K (forced-acceptance tests).
 */
size_t medusa_step_workspace_size(const medusa_model* m, const medusa_tree* t, int B, int64_t L_hint);
int medusa_step(const medusa_model* m, const medusa_tree* t, int B, int mode, float temperature, float eps,
                float delta, medusa_state* st, int64_t L_hint, const int32_t* topk_override, void* ws,
                size_t ws_bytes, hipStream_t stream);

/*
 * Fused draft + verify (page "大模型推理 memory bandwidth bound (5) - Medusa",
 * sections 二.5 and 二.7: the Medusa heads run on every tree position in the
 * verify pass, and the next candidates are taken at the accepted position,
 * medusa_logits[:, best, accept_length]).  One step: candidates from
 * topk_carry [B, H, K] int32 (device, caller-owned; in: this step's per-head
 * top-K, e.g. medusa_heads_topk on h_sel after prefill), the verify forward,
 * the heads and their top-K on all B*T tree nodes' final hidden states,
 * acceptance, KV compaction, and out: topk_carry = the top-K at each sequence's
 * selected node.  The state is updated as by medusa_step (h_sel included), so
 * both kinds of step can follow each other.  Same tokens as medusa_step under
 * greedy acceptance (both equal plain greedy decoding); the candidates can
 * differ from medusa_step's where the heads' products at B*T rows and at B rows
 * round differently.  Workspace: medusa_step_fused_workspace_size.  Errors as
 * medusa_step.
 */
size_t medusa_step_fused_workspace_size(const medusa_model* m, const medusa_tree* t, int B, int64_t L_hint);
int medusa_step_fused(const medusa_model* m, const medusa_tree* t, int B, int mode, float temperature, float eps,
                      float delta, medusa_state* st, int32_t* topk_carry, int64_t L_hint, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * The same step captured once into a HIP graph (all arguments, including the
 * state and workspace pointers, are baked in); medusa_graph_launch replays it on
 * any stream.  Capture needs a non-default stream.  Replays of one graph must not
 * overlap each other or other work on the same state.
 */
typedef struct medusa_graph medusa_graph;
int medusa_step_graph_create(const medusa_model* m, const medusa_tree* t, int B, int mode, float temperature,
                             float eps, float delta, medusa_state* st, int64_t L_hint, const int32_t* topk_override,
                             void* ws, size_t ws_bytes, hipStream_t stream, medusa_graph** out);
int medusa_graph_launch(medusa_graph* g, hipStream_t stream);
int medusa_graph_destroy(medusa_graph* g);

#ifdef __cplusplus
}
#endif
#endif /* MEDUSA_MODEL_H */
