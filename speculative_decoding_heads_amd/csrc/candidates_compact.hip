// Candidate expansion and KV compaction.
//
// tree_build_candidates follows generate_candidates() and the positions of
// tree_decoding() on the page "大模型推理 memory bandwidth bound (5) - Medusa"
// (sections 二.4, 二.5); kv_compact follows update_inference_inputs() (section
// 二.7), with the tree's K/V read from a side buffer so the copy never overlaps
// its own source.
#include "common.h"
#include "tree_dev.h"

using namespace medusa;

namespace {

// One block per sequence; thread i < T fills node i, threads also fill cart.
__global__ void candidates_kernel(const medusa_tree_host* __restrict__ t, int H, int K,
                                  const int32_t* __restrict__ root, const int32_t* __restrict__ topk,
                                  const int32_t* __restrict__ seq_len, int32_t* __restrict__ tree_tokens,
                                  int32_t* __restrict__ tree_pos, int32_t* __restrict__ cart) {
  __shared__ int32_t tok[MEDUSA_MAX_TREE];
  const int b = blockIdx.x;
  const int T = t->T, P = t->P, W = t->D + 1;
  const int tid = threadIdx.x;
  if (tid < T) {
    const int fi = t->tree_indices[tid];
    const int v = fi == 0 ? root[b] : topk[(size_t)b * H * K + (fi - 1)];
    tok[tid] = v;
    tree_tokens[(size_t)b * T + tid] = v;
    tree_pos[(size_t)b * T + tid] = seq_len[b] + t->depth[tid];
  }
  __syncthreads();
  for (int e = tid; e < P * W; e += blockDim.x) {
    const int p = e / W, j = e % W;
    const int node = t->retrieve[p * MEDUSA_MAX_TREE + j];
    cart[(size_t)b * P * W + e] = node >= 0 ? tok[node] : 0;
  }
}

// grid (n_layers * Hkv, B, 2 [K or V]); block handles up to D+1 rows of Dh
// elements with 16-byte moves.  Reads the pre-update seq_len.
template <int EB>
__global__ void compact_kv_kernel(const medusa_tree_host* __restrict__ t, int B, int Hkv, int Dh, int64_t Lmax,
                                  char* __restrict__ Kc, char* __restrict__ Vc, const char* __restrict__ Kt,
                                  const char* __restrict__ Vt, const int32_t* __restrict__ best,
                                  const int32_t* __restrict__ accept_len, const int32_t* __restrict__ seq_len,
                                  const int32_t* __restrict__ n_out, int max_new, int have_out) {
  const int lh = blockIdx.x;  // layer * Hkv + h
  const int b = blockIdx.y;
  const int layer = lh / Hkv, h = lh % Hkv;
  const int a = accept_len[b];
  const int s = seq_len[b];
  const int bi = best[b];
  if (a < 0 || bi < 0 || bi >= t->P || a + 1 > t->path_len[bi]) return;
  if ((int64_t)s + a + 1 > Lmax || s < 0) return;
  if (have_out && (n_out[b] < 0 || n_out[b] + a + 1 > max_new)) return;
  const int T = t->T;
  char* dst = blockIdx.z == 0 ? Kc : Vc;
  const char* src = blockIdx.z == 0 ? Kt : Vt;
  const size_t row_bytes = (size_t)Dh * EB;
  const size_t slab = ((size_t)layer * B + b) * Hkv + h;
  const size_t chunks = row_bytes / 16;
  for (size_t e = threadIdx.x; e < (size_t)(a + 1) * chunks; e += blockDim.x) {
    const int i = (int)(e / chunks);
    const size_t c = e % chunks;
    const int node = t->retrieve[bi * MEDUSA_MAX_TREE + i];
    const uint4* sp = (const uint4*)(src + (slab * T + node) * row_bytes) + c;
    uint4* dp = (uint4*)(dst + (slab * Lmax + s + i) * row_bytes) + c;
    *dp = *sp;
  }
}

// One thread per sequence: append tokens, bump lengths, flag overflow.
__global__ void compact_finalize_kernel(const medusa_tree_host* __restrict__ t, int B, int64_t Lmax,
                                        const int32_t* __restrict__ best, const int32_t* __restrict__ accept_len,
                                        int32_t* __restrict__ seq_len, const int32_t* __restrict__ tree_tokens,
                                        int32_t* __restrict__ out_tokens, int max_new, int32_t* __restrict__ n_out,
                                        int32_t* __restrict__ err_flag, int32_t* __restrict__ appended) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int a = accept_len[b];
  const int s = seq_len[b];
  const int bi = best[b];
  bool bad = a < 0 || bi < 0 || bi >= t->P || a + 1 > t->path_len[bi] || s < 0 || (int64_t)s + a + 1 > Lmax;
  if (!bad && out_tokens) bad = n_out[b] < 0 || n_out[b] + a + 1 > max_new;
  if (appended) appended[b] = bad ? 0 : 1;
  if (bad) {
    if (err_flag) *err_flag = 1;
    return;
  }
  if (out_tokens) {
    const int n = n_out[b];
    for (int i = 0; i <= a; ++i)
      out_tokens[(size_t)b * max_new + n + i] = tree_tokens[(size_t)b * t->T + t->retrieve[bi * MEDUSA_MAX_TREE + i]];
    n_out[b] = n + a + 1;
  }
  seq_len[b] = s + a + 1;
}

// Per-sequence stop: the number of this step's accepted tokens a sequence
// appends -- up to and including the first stop token (stop >= 0), and no
// more than its output room (max_new - n) and cache room (Lmax - s); fin is set
// when it appends the stop token or uses up a room.  The page's generation
// loop (section 二.1) ends once the end-of-sequence token is among the new
// tokens; a batch keeps its shape, so a finished sequence appends nothing more.
__device__ __forceinline__ int appended_count(const medusa_tree_host* t, const int32_t* tree_tokens, int b, int a,
                                              int bi, int s, int n, int max_new, int64_t Lmax, int stop, bool& fin) {
  int c = a + 1;
  fin = false;
  if (stop >= 0)
    for (int i = 0; i <= a; ++i)
      if (tree_tokens[(size_t)b * t->T + t->retrieve[bi * MEDUSA_MAX_TREE + i]] == stop) {
        c = i + 1;
        fin = true;
        break;
      }
  const int64_t room64 = min((int64_t)max_new - n, Lmax - s);
  const int room = (int)max<int64_t>(room64, 0);
  if (c >= room) {
    c = room;
    fin = true;
  }
  return c;
}

__device__ __forceinline__ bool compact_bad(const medusa_tree_host* t, int a, int bi, int s, int n) {
  return a < 0 || bi < 0 || bi >= t->P || a + 1 > t->path_len[bi] || s < 0 || n < 0;
}

template <int EB>
__global__ void compact_kv_stop_kernel(const medusa_tree_host* __restrict__ t, int B, int Hkv, int Dh, int64_t Lmax,
                                       char* __restrict__ Kc, char* __restrict__ Vc, const char* __restrict__ Kt,
                                       const char* __restrict__ Vt, const int32_t* __restrict__ best,
                                       const int32_t* __restrict__ accept_len, const int32_t* __restrict__ seq_len,
                                       const int32_t* __restrict__ tree_tokens, const int32_t* __restrict__ n_out,
                                       int max_new, const int32_t* __restrict__ done, int stop) {
  const int lh = blockIdx.x;  // layer * Hkv + h
  const int b = blockIdx.y;
  const int layer = lh / Hkv, h = lh % Hkv;
  if (done[b]) return;
  const int a = accept_len[b], s = seq_len[b], bi = best[b], n = n_out[b];
  if (compact_bad(t, a, bi, s, n)) return;
  bool fin;
  const int c = appended_count(t, tree_tokens, b, a, bi, s, n, max_new, Lmax, stop, fin);
  const int T = t->T;
  char* dst = blockIdx.z == 0 ? Kc : Vc;
  const char* src = blockIdx.z == 0 ? Kt : Vt;
  const size_t row_bytes = (size_t)Dh * EB;
  const size_t slab = ((size_t)layer * B + b) * Hkv + h;
  const size_t chunks = row_bytes / 16;
  for (size_t e = threadIdx.x; e < (size_t)c * chunks; e += blockDim.x) {
    const int i = (int)(e / chunks);
    const size_t ch = e % chunks;
    const int node = t->retrieve[bi * MEDUSA_MAX_TREE + i];
    *((uint4*)(dst + (slab * Lmax + s + i) * row_bytes) + ch) = *((const uint4*)(src + (slab * T + node) * row_bytes) + ch);
  }
}

__global__ void compact_stop_finalize_kernel(const medusa_tree_host* __restrict__ t, int B, int64_t Lmax,
                                             const int32_t* __restrict__ best, const int32_t* __restrict__ accept_len,
                                             int32_t* __restrict__ seq_len, const int32_t* __restrict__ tree_tokens,
                                             int32_t* __restrict__ out_tokens, int max_new, int32_t* __restrict__ n_out,
                                             int32_t* __restrict__ done, int stop, int32_t* __restrict__ err_flag,
                                             int32_t* __restrict__ appended) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  if (done[b]) {
    if (appended) appended[b] = 0;
    return;
  }
  const int a = accept_len[b], s = seq_len[b], bi = best[b], n = n_out[b];
  if (compact_bad(t, a, bi, s, n)) {
    if (appended) appended[b] = 0;
    if (err_flag) *err_flag = 1;
    return;
  }
  bool fin;
  const int c = appended_count(t, tree_tokens, b, a, bi, s, n, max_new, Lmax, stop, fin);
  // the next root and heads' input belong to the node after the last accepted
  // token: kept only when every accepted token was appended
  if (appended) appended[b] = c == a + 1 ? 1 : 0;
  for (int i = 0; i < c; ++i)
    out_tokens[(size_t)b * max_new + n + i] = tree_tokens[(size_t)b * t->T + t->retrieve[bi * MEDUSA_MAX_TREE + i]];
  n_out[b] = n + c;
  seq_len[b] = s + c;
  if (fin) done[b] = 1;
}

}  // namespace

extern "C" int tree_build_candidates(const medusa_tree* t, int B, int H, int K, const int32_t* root,
                                     const int32_t* topk_idx, const int32_t* seq_len, int32_t* tree_tokens,
                                     int32_t* tree_pos, int32_t* cart, hipStream_t stream) {
  MEDUSA_REQUIRE(B >= 0, MEDUSA_ERR_ARG, "tree_build_candidates: B < 0");
  MEDUSA_REQUIRE(t, MEDUSA_ERR_ARG, "tree_build_candidates: null tree");
  MEDUSA_REQUIRE(H >= t->host.D, MEDUSA_ERR_ARG, "tree_build_candidates: H=%d < tree depth %d", H, t->host.D);
  MEDUSA_REQUIRE(K == t->host.K, MEDUSA_ERR_ARG, "tree_build_candidates: K=%d but the tree uses %d", K,
                 t->host.K);
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(root && topk_idx && seq_len && tree_tokens && tree_pos && cart, MEDUSA_ERR_ARG,
                 "tree_build_candidates: null pointer");
  hipLaunchKernelGGL(candidates_kernel, dim3(B), dim3(64), 0, stream, t->dev, H, K, root, topk_idx, seq_len,
                     tree_tokens, tree_pos, cart);
  return check_launch("tree_build_candidates");
}

namespace medusa {
int kv_compact_flags(int dtype, const medusa_tree* t, int n_layers, int B, int Hkv, int Dh, int64_t Lmax, void* Kc,
                     void* Vc, const void* Kt, const void* Vt, const int32_t* best, const int32_t* accept_len,
                     int32_t* seq_len, const int32_t* tree_tokens, int32_t* out_tokens, int max_new, int32_t* n_out,
                     int32_t* err_flag, int32_t* appended, hipStream_t stream) {
  MEDUSA_REQUIRE(dtype_ok(dtype), MEDUSA_ERR_UNSUPPORTED, "kv_compact: dtype %d", dtype);
  MEDUSA_REQUIRE(n_layers >= 0 && B >= 0 && Hkv > 0 && Dh > 0 && Lmax > 0, MEDUSA_ERR_ARG, "kv_compact: bad sizes");
  MEDUSA_REQUIRE(((size_t)Dh * dtype_size(dtype)) % 16 == 0, MEDUSA_ERR_UNSUPPORTED,
                 "kv_compact: a K/V row must be a multiple of 16 bytes");
  MEDUSA_REQUIRE(!out_tokens || (n_out && max_new > 0), MEDUSA_ERR_ARG, "kv_compact: out_tokens needs n_out");
  MEDUSA_REQUIRE(t, MEDUSA_ERR_ARG, "kv_compact: null tree");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(best && accept_len && seq_len && tree_tokens, MEDUSA_ERR_ARG, "kv_compact: null pointer");
  if (n_layers > 0) {
    MEDUSA_REQUIRE(Kc && Vc && Kt && Vt, MEDUSA_ERR_ARG, "kv_compact: null K/V pointer");
    dim3 grid(n_layers * Hkv, B, 2);
    if (dtype == MEDUSA_BF16)
      hipLaunchKernelGGL(compact_kv_kernel<2>, grid, dim3(128), 0, stream, t->dev, B, Hkv, Dh, Lmax, (char*)Kc,
                         (char*)Vc, (const char*)Kt, (const char*)Vt, best, accept_len, seq_len, n_out, max_new,
                         out_tokens != nullptr);
    else
      hipLaunchKernelGGL(compact_kv_kernel<4>, grid, dim3(128), 0, stream, t->dev, B, Hkv, Dh, Lmax, (char*)Kc,
                         (char*)Vc, (const char*)Kt, (const char*)Vt, best, accept_len, seq_len, n_out, max_new,
                         out_tokens != nullptr);
    int rc = check_launch("kv_compact");
    if (rc) return rc;
  }
  hipLaunchKernelGGL(compact_finalize_kernel, dim3((B + 63) / 64), dim3(64), 0, stream, t->dev, B, Lmax, best,
                     accept_len, seq_len, tree_tokens, out_tokens, max_new, n_out, err_flag, appended);
  return check_launch("kv_compact finalize");
}

int kv_compact_stop(int dtype, const medusa_tree* t, int n_layers, int B, int Hkv, int Dh, int64_t Lmax, void* Kc,
                    void* Vc, const void* Kt, const void* Vt, const int32_t* best, const int32_t* accept_len,
                    int32_t* seq_len, const int32_t* tree_tokens, int32_t* out_tokens, int max_new, int32_t* n_out,
                    int32_t* done, int stop_token, int32_t* err_flag, int32_t* appended, hipStream_t stream) {
  MEDUSA_REQUIRE(t && dtype_ok(dtype), MEDUSA_ERR_ARG, "kv_compact_stop: bad tree or dtype");
  MEDUSA_REQUIRE(n_layers >= 0 && B >= 0 && Hkv > 0 && Dh > 0 && Lmax > 0, MEDUSA_ERR_ARG,
                 "kv_compact_stop: bad sizes");
  MEDUSA_REQUIRE(((size_t)Dh * dtype_size(dtype)) % 16 == 0, MEDUSA_ERR_UNSUPPORTED,
                 "kv_compact_stop: a K/V row must be a multiple of 16 bytes");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(best && accept_len && seq_len && tree_tokens && out_tokens && n_out && done && max_new > 0,
                 MEDUSA_ERR_ARG, "kv_compact_stop: null pointer");
  if (n_layers > 0) {
    MEDUSA_REQUIRE(Kc && Vc && Kt && Vt, MEDUSA_ERR_ARG, "kv_compact_stop: null K/V pointer");
    dim3 grid(n_layers * Hkv, B, 2);
    if (dtype == MEDUSA_BF16)
      hipLaunchKernelGGL(compact_kv_stop_kernel<2>, grid, dim3(128), 0, stream, t->dev, B, Hkv, Dh, Lmax, (char*)Kc,
                         (char*)Vc, (const char*)Kt, (const char*)Vt, best, accept_len, seq_len, tree_tokens, n_out,
                         max_new, done, stop_token);
    else
      hipLaunchKernelGGL(compact_kv_stop_kernel<4>, grid, dim3(128), 0, stream, t->dev, B, Hkv, Dh, Lmax, (char*)Kc,
                         (char*)Vc, (const char*)Kt, (const char*)Vt, best, accept_len, seq_len, tree_tokens, n_out,
                         max_new, done, stop_token);
    int rc = check_launch("kv_compact_stop");
    if (rc) return rc;
  }
  hipLaunchKernelGGL(compact_stop_finalize_kernel, dim3((B + 63) / 64), dim3(64), 0, stream, t->dev, B, Lmax, best,
                     accept_len, seq_len, tree_tokens, out_tokens, max_new, n_out, done, stop_token, err_flag,
                     appended);
  return check_launch("kv_compact_stop finalize");
}

}  // namespace medusa

extern "C" int kv_compact(int dtype, const medusa_tree* t, int n_layers, int B, int Hkv, int Dh, int64_t Lmax,
                          void* Kc, void* Vc, const void* Kt, const void* Vt, const int32_t* best,
                          const int32_t* accept_len, int32_t* seq_len, const int32_t* tree_tokens,
                          int32_t* out_tokens, int max_new, int32_t* n_out, int32_t* err_flag,
                          hipStream_t stream) {
  return kv_compact_flags(dtype, t, n_layers, B, Hkv, Dh, Lmax, Kc, Vc, Kt, Vt, best, accept_len, seq_len,
                          tree_tokens, out_tokens, max_new, n_out, err_flag, nullptr, stream);
}

