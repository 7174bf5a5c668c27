/*
 * medusa.h -- C ABI of libmedusa: one Medusa verify iteration on an AMD
 * Instinct MI355X (gfx950), as hand-written HIP kernels.
 *
 * The method is the one described on the page "大模型推理 memory bandwidth
 * bound (5) - Medusa" (section 一: Medusa heads, tree attention, typical
 * acceptance; section 二: generate_medusa_buffers, generate_candidates,
 * tree_decoding, evaluate_posterior, update_inference_inputs), and on
 * "基于 Medusa 投机解码的 OpenPangu-7B 在 Ascend NPU 的推理加速实现" (section 2:
 * heads propose, a candidate tree is built, tree attention verifies all
 * candidates in one pass, the longest acceptable prefix is kept).
 *
 * Conventions shared by every call
 *  - Return value: MEDUSA_OK (0) or a negative MEDUSA_ERR_* code; the message of
 *    the last failure on the calling thread is medusa_last_error().  Nothing is
 *    launched when a call returns an error, and no C++ exception crosses the ABI.
 *  - Tensor pointers are DEVICE pointers owned by the caller, contiguous,
 *    row-major in the layouts stated per argument.  Host pointers are marked.
 *  - bf16 tensors hold IEEE bfloat16 bit patterns (uint16 storage).
 *  - Device calls only enqueue work on `stream` and never synchronise.  Scratch
 *    memory comes from a caller-provided workspace whose minimum size is given
 *    by the matching *_workspace_size() query; the library allocates nothing in
 *    these calls (device memory is allocated only by medusa_tree_create).
 *  - Values that live on the device (sequence lengths, accepted lengths) are
 *    not validated on the host; kernels clamp reads to the buffers they were
 *    given and report overflow through an error flag where stated.
 */
#ifndef MEDUSA_H
#define MEDUSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MEDUSA_OK = 0,
  MEDUSA_ERR_ARG = -1,          /* a null pointer, a bad size, an inconsistent shape */
  MEDUSA_ERR_UNSUPPORTED = -2,  /* valid but not implemented (dtype, head size, tree size) */
  MEDUSA_ERR_WORKSPACE = -3,    /* workspace smaller than the *_workspace_size() query */
  MEDUSA_ERR_HIP = -4           /* a HIP runtime call or launch failed */
};

enum { MEDUSA_F32 = 0, MEDUSA_BF16 = 1 };
enum { MEDUSA_GREEDY = 0, MEDUSA_TYPICAL = 1, MEDUSA_SAMPLED = 2 };
enum { MEDUSA_SAMPLE_TYPICAL = 1, MEDUSA_SAMPLE_NUCLEUS = 2 };

#define MEDUSA_MAX_TREE 64 /* nodes per tree, root included: one 64-bit mask word per node */

const char* medusa_last_error(void);
int medusa_version(void);

/* ------------------------------------------------------------------------- */
/* Static tree                                                                */
/* ------------------------------------------------------------------------- */
/*
 * Host copy of the buffers generate_medusa_buffers() derives from the choice
 * list (page "memory bandwidth bound (5) - Medusa", section 二.2):
 *   nodes sorted by (depth, ranks), node 0 = root;
 *   tree_indices[i] = 1 + K*(depth-1) + last rank  (index into the flat list
 *                     [root, head1 top-K, ..., headH top-K]);
 *   depth[i]        = medusa_position_ids;
 *   anc[i]          = bit j set iff node j is an ancestor of i or i itself
 *                     (the row of medusa_attn_mask as a bitset);
 *   retrieve[p][j]  = retrieve_indices, one row per leaf in decreasing leaf
 *                     index, -1 padded; row stride MEDUSA_MAX_TREE;
 *   path_len[p]     = number of non-pad entries of row p.
 */
typedef struct medusa_tree_host {
  int32_t T, D, P, K, H;  /* nodes, max depth, paths, top-K stride, heads used (= D) */
  int32_t tree_indices[MEDUSA_MAX_TREE];
  int32_t depth[MEDUSA_MAX_TREE];
  int32_t parent[MEDUSA_MAX_TREE];
  int32_t path_len[MEDUSA_MAX_TREE];
  uint64_t anc[MEDUSA_MAX_TREE];
  int32_t retrieve[MEDUSA_MAX_TREE * MEDUSA_MAX_TREE];
} medusa_tree_host;

typedef struct medusa_tree medusa_tree; /* opaque: host copy + device copy */

/*
 * Build and validate a tree from a flattened choice list and upload it to the
 * current device.  ranks (host) holds the rank paths back to back; choice c is
 * ranks[offsets[c] .. offsets[c+1]).  K = top-K stride, or <= 0 for "1 + the
 * largest rank used".  Rejects (MEDUSA_ERR_ARG): duplicates, a choice whose
 * parent is absent, negative ranks, rank >= K; (MEDUSA_ERR_UNSUPPORTED): more
 * than MEDUSA_MAX_TREE nodes.  Allocates device memory (setup, not hot path).
 */
int medusa_tree_create(const int32_t* ranks, const int32_t* offsets, int32_t n_choices, int32_t K,
                       medusa_tree** out);
/* The same construction and validation on the host only (no device memory). */
int medusa_tree_build_host(const int32_t* ranks, const int32_t* offsets, int32_t n_choices, int32_t K,
                           medusa_tree_host* out);
/* Copy the host-side buffers (for inspection and tests). */
int medusa_tree_info(const medusa_tree* t, medusa_tree_host* out);
/* Device pointer to the tree's anc[] words (uint64[T]) for tree_attention. */
const uint64_t* medusa_tree_anc_device(const medusa_tree* t);
int medusa_tree_destroy(medusa_tree* t);

/* ------------------------------------------------------------------------- */
/* The five calls of the verify iteration                                     */
/* ------------------------------------------------------------------------- */

/*
 * Medusa heads + per-head top-K (page "memory bandwidth bound (5) - Medusa",
 * section 一.1: p^(k) = softmax(W2^(k) (SiLU(W1^(k) h) + h)), and section 二.4:
 * candidates are torch.topk(medusa_logits, K).indices).
 *   h        [B, d]        dtype   hidden state the heads read (final-normed)
 *   W1       [H, d, d]     dtype   row j of W1[k] produces output j
 *   W2       [H, V, d]     dtype   stored V x d: logits = W2 z
 *   topk_idx [B, H, K]     int32   value-descending; ties -> lower token index
 *   topk_val [B, H, K]     float   logits at topk_idx (nullable)
 * The residual output z = h + SiLU(W1 h) is stored in `dtype` before the
 * V-projection; logits are fp32.  K <= 16.
 */
size_t medusa_heads_topk_workspace_size(int dtype, int B, int d, int V, int H, int K);
int medusa_heads_topk(int dtype, int B, int d, int V, int H, int K, const void* h, const void* W1,
                      const void* W2, int32_t* topk_idx, float* topk_val, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * Candidate expansion (section 二.4 generate_candidates, section 二.5 positions):
 *   root        [B]            int32   the greedy root token of each sequence
 *   topk_idx    [B, H, K]      int32   H = tree heads used (>= t's depth), K = t's stride
 *   seq_len     [B]            int32   current sequence length (tokens in the KV cache)
 *   tree_tokens [B, T]         int32   flat[tree_indices], flat = [root, topk_idx[b].ravel()]
 *   tree_pos    [B, T]         int32   seq_len + depth
 *   cart        [B, P, D+1]    int32   tree_tokens gathered by retrieve_indices, pad -> 0
 */
int tree_build_candidates(const medusa_tree* t, int B, int H, int K, const int32_t* root,
                          const int32_t* topk_idx, const int32_t* seq_len, int32_t* tree_tokens,
                          int32_t* tree_pos, int32_t* cart, hipStream_t stream);

/*
 * Tree attention (section 一.2: the tree is flattened into one sequence and a
 * node only attends to its predecessors; section 二.2 medusa_attn_mask; every
 * cached prefix token is visible to every node).  For tree node i and query
 * head h (KV head h / (Hq/Hkv)):
 *   out[b,i,h] = softmax(scale * q.k over prefix rows 0..seq_len[b]-1 of Kc and
 *                the tree rows j of Kt with bit j of anc[i]) @ the same rows of V.
 *   q      [B, T, Hq, Dh]       dtype
 *   Kc, Vc [B, Hkv, Lmax, Dh]   dtype   KV cache; rows >= seq_len[b] are never read
 *   Kt, Vt [B, Hkv, T, Dh]      dtype   the tree tokens' own K/V
 *   anc    [T]                  uint64  device; bit j of anc[i] = node j visible to i
 *   out    [B, T, Hq, Dh]       dtype
 *   L_hint  host upper bound of max(seq_len) used to size the split-KV grid (<= Lmax)
 * T <= 64.  bf16 with Dh in {64, 128}: the MFMA kernel; fp32, and bf16 with
 * any other Dh <= 128: the generic kernel (deterministic key order by absolute
 * position); Dh > 128 outside {64, 128} returns MEDUSA_ERR_UNSUPPORTED.
 * Also serves chain-masked prefill chunks (anc = lower triangle) and T = 1 decode.
 */
size_t tree_attention_workspace_size(int dtype, int B, int T, int Hq, int Hkv, int Dh, int64_t L_hint);
int tree_attention(int dtype, int B, int T, int Hq, int Hkv, int Dh, const void* q, const void* Kc,
                   const void* Vc, int64_t Lmax, int64_t L_hint, const int32_t* seq_len, const void* Kt,
                   const void* Vt, const uint64_t* anc, float scale, void* out, void* ws, size_t ws_bytes,
                   hipStream_t stream);

/*
 * tree_attention without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, serving loops that forbid
 * allocation).  Same arguments, kernels and results as tree_attention; the split
 * partials go to a fixed array inside the library (tree_attention_noalloc_max_scratch()
 * bytes, 64 MiB, held on every device the library runs on until the process
 * ends).  A shape whose tree_attention_workspace_size exceeds that returns
 * MEDUSA_ERR_WORKSPACE before anything is launched.  Nothing in the array needs
 * clearing between calls; every call on one device shares it, so calls that
 * overlap on one device (different streams, or graphs replayed concurrently)
 * race and must be serialised by the caller.
 */
size_t tree_attention_noalloc_max_scratch(void);
int tree_attention_noalloc(int dtype, int B, int T, int Hq, int Hkv, int Dh, const void* q, const void* Kc,
                           const void* Vc, int64_t Lmax, int64_t L_hint, const int32_t* seq_len, const void* Kt,
                           const void* Vt, const uint64_t* anc, float scale, void* out, hipStream_t stream);

/*
 * Acceptance (section 二.6 evaluate_posterior, section 一.3 typical acceptance):
 *   GREEDY : candidate accepted iff it equals argmax of its parent's logits.
 *   TYPICAL: q = softmax(logits/temperature) at the parent, H = -sum q log(q+1e-5),
 *            accepted iff q(candidate) > min(eps, delta*exp(-H)).
 * Per path: leading accepted count (pads never accepted); a = max; best = 0 if
 * a == 0, else first path of length a (GREEDY) or, among them, the largest sum
 * of log q of the accepted candidates, first on ties (TYPICAL).
 *   logits      [B, T, V]  float   LM-head logits of every tree node
 *   tree_tokens [B, T]     int32
 *   best, accept_len, sel_node (= retrieve[best][a]), next_root (= argmax at sel_node)  [B] int32
 */
size_t evaluate_posterior_workspace_size(int B, int T);
int evaluate_posterior(const medusa_tree* t, int B, int V, const float* logits, const int32_t* tree_tokens,
                       int mode, float temperature, float eps, float delta, int32_t* best,
                       int32_t* accept_len, int32_t* sel_node, int32_t* next_root, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * State update (section 二.7 update_inference_inputs), all layers in one call:
 *   for i in 0..a_b: Kc/Vc[l, b, h, seq_len[b]+i, :] = Kt/Vt[l, b, h, retrieve[best_b][i], :]
 *   out_tokens[b, n_out[b]+i] = tree_tokens[b, retrieve[best_b][i]]
 *   seq_len[b] += a_b + 1;  n_out[b] += a_b + 1
 *   Kc, Vc [n_layers, B, Hkv, Lmax, Dh]   Kt, Vt [n_layers, B, Hkv, T, Dh]   dtype
 *   out_tokens [B, max_new] int32 (nullable, then n_out is ignored)
 * If seq_len + a + 1 > Lmax or n_out + a + 1 > max_new for a sequence, nothing is
 * written for it and *err_flag (device int32, nullable) is set to 1.
 */
int kv_compact(int dtype, const medusa_tree* t, int n_layers, int B, int Hkv, int Dh, int64_t Lmax,
               void* Kc, void* Vc, const void* Kt, const void* Vt, const int32_t* best,
               const int32_t* accept_len, int32_t* seq_len, const int32_t* tree_tokens,
               int32_t* out_tokens, int max_new, int32_t* n_out, int32_t* err_flag, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Sampling: the sampled root and the non-fast acceptance branch              */
/* ------------------------------------------------------------------------- */
/*
 * Page "memory bandwidth bound (5) - Medusa": generate_candidates() (section
 * 二.4) draws the root with get_typical_one_token / get_nucleus_one_token unless
 * the temperature is 0 or `fast` is set (top_p defaults to 0.8, section 二.1);
 * section 一.3 gives the typical allow set {x : p(x) > min(eps, delta exp(-H))};
 * evaluate_posterior() (section 二.6) outside the fast branch keeps the first
 * path of the longest accepted length.  The pages do not print those bodies;
 * the reading implemented:
 *   q = softmax(logits / temperature).  TYPICAL keeps {q > eta}, eta =
 *   min(eps, delta exp(-H)), H = -sum q log(q + 1e-5) (an empty set leaves the
 *   argmax); NUCLEUS keeps the smallest set of the most probable tokens whose
 *   mass reaches top_p, ties with the last one included.  A draw is the allowed
 *   token with the largest log q(x) - log(-log U(x)) (Gumbel-max; lowest index on
 *   ties), U from Philox4x32-10 keyed by `seed`, counter (x / 4, position,
 *   sequence, 0), output word x % 4, U = (2 (r >> 9) + 1) / 2^24.  `position`
 *   is the absolute position of the token whose logits are sampled.
 */
typedef struct medusa_sampling {
  int32_t kind;      /* MEDUSA_SAMPLE_TYPICAL or MEDUSA_SAMPLE_NUCLEUS */
  float temperature; /* > 0 */
  float eps, delta;  /* typical: posterior_threshold, posterior_alpha */
  float top_p;       /* nucleus */
  uint64_t seed;
} medusa_sampling;

/*
 * One draw per row: out[r] drawn from logits[r*ldx .. r*ldx + V) (fp32, device)
 * for sequence seq_id[r] (nullable: r) at position pos[r] (device int32 [M]).
 * s is a host pointer read at the call.
 */
int medusa_sample_tokens(const medusa_sampling* s, int M, int V, const float* logits, int64_t ldx,
                         const int32_t* seq_id, const int32_t* pos, int32_t* out, hipStream_t stream);

/*
 * Non-fast acceptance: one draw at every tree node u of sequence b (its logits
 * row, position tree_pos[b, u], sequence b); a candidate is accepted when its
 * token equals the draw at its parent (pads never); best = the first path of the
 * longest accepted length (0 when none); sel_node = retrieve[best][a];
 * next_root = the draw at sel_node.  Outputs and layouts as evaluate_posterior;
 * tree_pos [B, T] int32 as tree_build_candidates writes it.
 */
size_t evaluate_posterior_sampled_workspace_size(int B, int T);
int evaluate_posterior_sampled(const medusa_tree* t, int B, int V, const float* logits, const int32_t* tree_tokens,
                               const int32_t* tree_pos, const medusa_sampling* s, int32_t* best,
                               int32_t* accept_len, int32_t* sel_node, int32_t* next_root, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Tree calibration                                                           */
/* ------------------------------------------------------------------------- */

/*
 * The static sparse tree from per-(depth, rank) acceptance rates (page
 * "memory bandwidth bound (5) - Medusa", section 一.2: the tree is built ahead
 * of time, keeping the probable candidate paths; the figure there relates the
 * candidate count to the accepted length and the speed).  Reading, as the page
 * gives no construction: the true token of depth d sits at rank r of head d's
 * top-K with probability acc[d*K + r], ranks of one depth exclusive, depths
 * independent; a path's probability is the product of acc along its ranks
 * (multiplied from depth 0 up); a tree's expected accepted length is the sum of
 * its paths' probabilities, which the n_nodes - 1 most probable paths maximise
 * (ties: the shorter path, then the lexicographically smaller ranks).
 *   acc        host, H*K doubles, each in [0, 1], each depth's sum <= 1
 *   n_nodes    1..MEDUSA_MAX_TREE nodes, root included, <= 1 + sum_d K^d
 *   ranks      host out, capacity (n_nodes - 1) * H: the paths' ranks, concatenated
 *   offsets    host out, n_nodes entries: path i = ranks[offsets[i] .. offsets[i+1])
 *              (the medusa_tree_create format), in selection order
 *   expected   host out (nullable): the sum of the chosen path probabilities,
 *              added in selection order
 * Host only (no device call).  MEDUSA_ERR_ARG for bad sizes or a bad table.
 */
int medusa_tree_from_acceptance(const double* acc, int32_t H, int32_t K, int32_t n_nodes, int32_t* ranks,
                                int32_t* offsets, double* expected);

/*
 * Teacher-forced hits of the heads, the measurement behind such a table: for
 * every position t < N and head k < H with t + k + 2 < n_tokens,
 *   positions[k] += 1;  counts[k*K + r] += (topk[(t*H + k)*K + r] == tokens[t + k + 2])
 * (head k at the hidden state of tokens[t] predicts the token k + 1 places
 * after the LM head's target tokens[t + 1]).
 *   topk [N, H, K] int32, tokens [n_tokens] int32: device
 *   counts [H*K], positions [H] int64: device, added to (the caller zeroes them)
 * H*K <= 4096.  Counts are exact integers, independent of the launch shape.
 */
int medusa_head_hits(int N, int H, int K, const int32_t* topk, const int32_t* tokens, int n_tokens,
                     int64_t* counts, int64_t* positions, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MEDUSA_H */
