// Medusa heads + per-head top-K.
//
// The page "大模型推理 memory bandwidth bound (5) - Medusa" defines a head as one
// residual block, p^(k) = softmax(W2^(k) (SiLU(W1^(k) h) + h)) (section 一.1),
// and generate_candidates() keeps the indices of each head's top-K logits
// (section 二.4; softmax is monotone, so the logits suffice).  The call runs
//   1. z = h + SiLU(W1 h) for all heads at once (W1 stacked [H*d, d]) with the
//      residual fused into the product's epilogue, z stored in the input dtype;
//   2. logits[b, k, :] = W2[k] z[b, k] as H batched products (fp32 out);
//   3. top-K per (b, k) row: each thread keeps a sorted register list over a
//      strided slice of the vocabulary, then K rounds of a block-wide
//      (value desc, index asc) maximum pop the winners.
#include "common.h"
#include "medusa_model.h"

using namespace medusa;

namespace {

constexpr int TK_MAX = 16;
constexpr int TK_THR = 256;

__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

__global__ __launch_bounds__(TK_THR) void topk_rows_kernel(int V, const float* __restrict__ x, int K,
                                                           int32_t* __restrict__ idx, float* __restrict__ val) {
  const int row = blockIdx.x;
  const float* r = x + (size_t)row * V;
  float lv[TK_MAX];
  int li[TK_MAX];
#pragma unroll
  for (int j = 0; j < TK_MAX; ++j) {
    lv[j] = -INFINITY;
    li[j] = 0x7fffffff;
  }
  for (int k = threadIdx.x; k < V; k += TK_THR) {
    const float v = r[k];
    if (!better(v, k, lv[TK_MAX - 1], li[TK_MAX - 1])) continue;
    lv[TK_MAX - 1] = v;
    li[TK_MAX - 1] = k;
#pragma unroll
    for (int j = TK_MAX - 1; j > 0; --j) {
      if (better(lv[j], li[j], lv[j - 1], li[j - 1])) {
        const float tv = lv[j];
        lv[j] = lv[j - 1];
        lv[j - 1] = tv;
        const int ti = li[j];
        li[j] = li[j - 1];
        li[j - 1] = ti;
      }
    }
  }
  __shared__ float sv[TK_THR / 64];
  __shared__ int si[TK_THR / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int round = 0; round < K; ++round) {
    float bv = lv[0];
    int bi = li[0];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o, 64);
      const int i2 = __shfl_xor(bi, o, 64);
      if (better(v2, i2, bv, bi)) {
        bv = v2;
        bi = i2;
      }
    }
    if (lane == 0) {
      sv[w] = bv;
      si[w] = bi;
    }
    __syncthreads();
    bv = sv[0];
    bi = si[0];
#pragma unroll
    for (int j = 1; j < TK_THR / 64; ++j)
      if (better(sv[j], si[j], bv, bi)) {
        bv = sv[j];
        bi = si[j];
      }
    __syncthreads();
    if (threadIdx.x == 0) {
      idx[(size_t)row * K + round] = bi == 0x7fffffff ? 0 : bi;
      if (val) val[(size_t)row * K + round] = bv;
    }
    if (li[0] == bi && bi != 0x7fffffff) {  // the owner pops its head
#pragma unroll
      for (int j = 0; j < TK_MAX - 1; ++j) {
        lv[j] = lv[j + 1];
        li[j] = li[j + 1];
      }
      lv[TK_MAX - 1] = -INFINITY;
      li[TK_MAX - 1] = 0x7fffffff;
    }
  }
}

struct HeadsLayout {
  size_t z_off, logits_off, gemm_off, total;
};

HeadsLayout heads_layout(int dtype, int B, int d, int V, int H) {
  HeadsLayout L;
  L.z_off = 0;
  L.logits_off = align_up((size_t)B * H * d * dtype_size(dtype), 256);
  L.gemm_off = L.logits_off + align_up((size_t)B * H * V * sizeof(float), 256);
  size_t g1 = medusa_gemm_workspace_size(dtype, B, H * d, d, 1);
  size_t g2 = medusa_gemm_workspace_size(dtype, B, V, d, H);
  L.total = L.gemm_off + (g1 > g2 ? g1 : g2);
  return L;
}

}  // namespace

extern "C" int medusa_topk_rows(int M, int V, const float* x, int K, int32_t* idx, float* val, hipStream_t stream) {
  MEDUSA_REQUIRE(M >= 0 && V > 0, MEDUSA_ERR_ARG, "topk_rows: bad sizes");
  MEDUSA_REQUIRE(K >= 1 && K <= TK_MAX && K <= V, MEDUSA_ERR_UNSUPPORTED, "topk_rows: K=%d not in [1, %d]", K, TK_MAX);
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(x && idx, MEDUSA_ERR_ARG, "topk_rows: null pointer");
  hipLaunchKernelGGL(topk_rows_kernel, dim3(M), dim3(TK_THR), 0, stream, V, x, K, idx, val);
  return check_launch("topk_rows");
}

extern "C" size_t medusa_heads_topk_workspace_size(int dtype, int B, int d, int V, int H, int K) {
  if (B <= 0 || d <= 0 || V <= 0 || H <= 0) return 0;
  return heads_layout(dtype, B, d, V, H).total;
}

extern "C" int medusa_heads_topk(int dtype, int B, int d, int V, int H, int K, const void* h, const void* W1,
                                 const void* W2, int32_t* topk_idx, float* topk_val, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  MEDUSA_REQUIRE(dtype_ok(dtype), MEDUSA_ERR_UNSUPPORTED, "heads_topk: dtype %d", dtype);
  MEDUSA_REQUIRE(B >= 0 && d > 0 && V > 0 && H > 0, MEDUSA_ERR_ARG, "heads_topk: bad sizes");
  MEDUSA_REQUIRE(K >= 1 && K <= TK_MAX && K <= V, MEDUSA_ERR_UNSUPPORTED, "heads_topk: K=%d not in [1, %d]", K,
                 TK_MAX);
  MEDUSA_REQUIRE(dtype == MEDUSA_F32 || d % 32 == 0, MEDUSA_ERR_UNSUPPORTED, "heads_topk: bf16 needs d %% 32 == 0");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(h && W1 && W2 && topk_idx, MEDUSA_ERR_ARG, "heads_topk: null pointer");
  HeadsLayout L = heads_layout(dtype, B, d, V, H);
  MEDUSA_REQUIRE(ws && ws_bytes >= L.total, MEDUSA_ERR_WORKSPACE, "heads_topk: workspace %zu < %zu", ws_bytes, L.total);
  char* base = (char*)ws;
  void* z = base + L.z_off;
  float* logits = (float*)(base + L.logits_off);
  void* gws = base + L.gemm_off;
  const size_t gbytes = ws_bytes - L.gemm_off;
  int rc = medusa_gemm(dtype, B, H * d, d, h, d, 0, W1, 0, z, (int64_t)H * d, 0, 1, MEDUSA_EPI_SILU_RESID_A, nullptr, 0,
                       0, gws, gbytes, stream);
  if (rc) return rc;
  rc = medusa_gemm(dtype, B, V, d, z, (int64_t)H * d, d, W2, (int64_t)V * d, logits, (int64_t)H * V, V, H,
                   MEDUSA_EPI_F32, nullptr, 0, 0, gws, gbytes, stream);
  if (rc) return rc;
  return medusa_topk_rows(B * H, V, logits, K, topk_idx, topk_val, stream);
}
