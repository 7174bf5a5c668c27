// Acceptance and longest-path selection.
//
// Follows evaluate_posterior() on the page "大模型推理 memory bandwidth bound (5)
// - Medusa" (section 二.6) and the typical-acceptance rule of section 一.3.  The
// page evaluates every root-to-leaf path on a [paths, depth, V] copy of the
// logits; here the per-node statistics are computed once per tree node (each
// node's logits are read from memory once per pass), and one lane per path then
// walks its path.
//
//   pass A, grid (T, B): per node u -- argmax (lowest index on ties); for
//     typical also max, Z = sum exp((x-max)/tau) and
//     H = -sum q log(q + 1e-5) with q = exp((x-max)/tau)/Z, threshold
//     thr = min(eps, delta*exp(-H)).
//   pass B, grid (B): lane p walks path p, counts leading accepted candidates
//     (pads never accepted), sums log q for typical; a wave reduction picks
//     the accept length, the best path, the selected node and the next root.
#include "common.h"
#include "tree_dev.h"

using namespace medusa;

namespace {

struct NodeStat {
  int32_t amax;
  float m, Z, thr;
};

constexpr int kStatThreads = 1024;

__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// NV > 0 (vec rows of at most NV * 4 * kStatThreads entries): the row is held in
// registers, NV float4 a thread, every load issued before the first use, and pass
// 2 reads no memory; NV == 0 streams the row twice (the second time from L2).
// Each thread visits its entries in the same order either way (thread tid owns
// float4 tid, tid + kStatThreads, ...), so the results are the same.  vec: the
// rows are 16-byte aligned (V % 4 == 0 and an aligned base).
template <int NV>
__global__ __launch_bounds__(kStatThreads) void node_stats_kernel(const float* __restrict__ logits, int T, int V,
                                                                 int vec, int typical, float inv_tau, float eps,
                                                                 float delta, NodeStat* __restrict__ out) {
  const int u = blockIdx.x, b = blockIdx.y;
  const float* x = logits + ((size_t)b * T + u) * V;
  const int tid = threadIdx.x;
  __shared__ float s_v[kStatThreads / 64];
  __shared__ int s_i[kStatThreads / 64];
  __shared__ float s_f[kStatThreads / 64];
  const int lane = tid & 63, w = tid >> 6;
  const int V4 = V / 4;
  float4 f[NV > 0 ? NV : 1];
  if constexpr (NV > 0) {
    const float4* x4 = (const float4*)x;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int k4 = tid + j * kStatThreads;
      f[j] = x4[k4 < V4 ? k4 : V4 - 1];  // a clamped index, not a branch: the loads go out together
    }
  }

  // pass 1: argmax, and for typical an online sum of exp((x - running max)/tau),
  // as 2^((x - max) * log2(e)/tau) on the hardware base-2 exponential
  const float c2 = inv_tau * 1.4426950408889634f;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  float z = 0.f;
  auto visit = [&](float v, int k) {
    if (v > bv) {  // strictly greater keeps the lowest index of this thread's stripe
      if (typical) z = z * __builtin_amdgcn_exp2f((bv - v) * c2) + 1.0f;
      bv = v;
      bi = k;
    } else if (typical) {
      z += __builtin_amdgcn_exp2f((v - bv) * c2);
    }
  };
  if constexpr (NV > 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int k4 = tid + j * kStatThreads;
      if (k4 < V4) {
        visit(f[j].x, 4 * k4);
        visit(f[j].y, 4 * k4 + 1);
        visit(f[j].z, 4 * k4 + 2);
        visit(f[j].w, 4 * k4 + 3);
      }
    }
  } else if (vec) {
    const float4* x4 = (const float4*)x;
    for (int k4 = tid; k4 < V4; k4 += kStatThreads) {
      const float4 g = x4[k4];
      visit(g.x, 4 * k4);
      visit(g.y, 4 * k4 + 1);
      visit(g.z, 4 * k4 + 2);
      visit(g.w, 4 * k4 + 3);
    }
  } else {
    for (int k = tid; k < V; k += kStatThreads) visit(x[k], k);
  }
  auto merge = [&](float v2, int i2, float z2) {
    const float m = fmaxf(bv, v2);
    if (typical && m != -INFINITY)
      z = z * __builtin_amdgcn_exp2f((bv - m) * c2) + z2 * __builtin_amdgcn_exp2f((v2 - m) * c2);
    argmax_merge(bv, bi, v2, i2);
  };
  butterfly([&](auto S) {
    constexpr int s = decltype(S)::value;
    merge(bfly<s>(bv), bfly<s>(bi), bfly<s>(z));
  });
  if (lane == 0) {
    s_v[w] = bv;
    s_i[w] = bi;
    s_f[w] = z;
  }
  __syncthreads();
  // wave 0 merges the waves' partials in wave order and shares the result (the
  // sixteen waves doing the same merge would share the four SIMDs)
  if (w == 0) {
    bv = s_v[0];
    bi = s_i[0];
    z = s_f[0];
    for (int j = 1; j < kStatThreads / 64; ++j) merge(s_v[j], s_i[j], s_f[j]);
    if (lane == 0) {
      s_v[0] = bv;
      s_i[0] = bi;
      s_f[0] = z;
    }
  }
  __syncthreads();
  bv = s_v[0];
  bi = s_i[0];
  z = s_f[0];
  if (bi == 0x7fffffff) bi = 0;  // all NaN row: report token 0
  if (!typical) {
    if (tid == 0) out[(size_t)b * T + u] = NodeStat{bi, bv, 0.f, 0.f};
    return;
  }
  const float m = bv;
  const float Z = z;
  const float invZ = 1.0f / Z;
  // pass 2: H = -sum q log(q + 1e-5), natural log as log2 * ln 2 (the ln 2 is
  // applied once to the sum)
  float hsum = 0.f;
  auto hterm = [&](float v) {
    const float q = __builtin_amdgcn_exp2f((v - m) * c2) * invZ;
    hsum += q * __builtin_amdgcn_logf(q + 1e-5f);
  };
  if constexpr (NV > 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int k4 = tid + j * kStatThreads;
      if (k4 < V4) {
        hterm(f[j].x);
        hterm(f[j].y);
        hterm(f[j].z);
        hterm(f[j].w);
      }
    }
  } else if (vec) {
    const float4* x4 = (const float4*)x;
    for (int k4 = tid; k4 < V4; k4 += kStatThreads) {
      const float4 g = x4[k4];
      hterm(g.x);
      hterm(g.y);
      hterm(g.z);
      hterm(g.w);
    }
  } else {
    for (int k = tid; k < V; k += kStatThreads) hterm(x[k]);
  }
  hsum = wave_sum(hsum);
  __syncthreads();
  if (lane == 0) s_f[w] = hsum;
  __syncthreads();
  if (tid == 0) {
    float hs = 0.f;
    for (int j = 0; j < kStatThreads / 64; ++j) hs += s_f[j];
    const float H = -hs * 0.6931471805599453f;
    const float thr = fminf(eps, delta * expf(-H));
    out[(size_t)b * T + u] = NodeStat{bi, m, Z, thr};
  }
}

// One wave per sequence, lane p = path p (P <= 64).
__global__ __launch_bounds__(64) void select_kernel(const medusa_tree_host* __restrict__ t, const float* __restrict__ logits,
                                                    int V, const int32_t* __restrict__ tree_tokens, int typical,
                                                    float inv_tau, const NodeStat* __restrict__ st,
                                                    int32_t* __restrict__ best_out, int32_t* __restrict__ acc_out,
                                                    int32_t* __restrict__ sel_out, int32_t* __restrict__ root_out) {
  const int b = blockIdx.x;
  const int p = threadIdx.x;
  const int T = t->T, P = t->P;
  const NodeStat* s = st + (size_t)b * T;
  int acc = -1;  // lanes without a path never win
  float lik = -INFINITY;
  if (p < P) {
    acc = 0;
    lik = 0.f;
    const int len = t->path_len[p];
    const int32_t* row = t->retrieve + p * MEDUSA_MAX_TREE;
    for (int j = 1; j < len; ++j) {
      const int u = row[j - 1];
      const int tok = tree_tokens[(size_t)b * T + row[j]];
      bool ok;
      if (!typical) {
        ok = tok == s[u].amax;
      } else {
        float q = 0.f;
        if (tok >= 0 && tok < V) q = expf((logits[((size_t)b * T + u) * V + tok] - s[u].m) * inv_tau) / s[u].Z;
        ok = q > s[u].thr;
        if (ok) lik += logf(q);
      }
      if (!ok) break;
      ++acc;
    }
  }
  // a = max acc
  int a = acc;
  a = wave_max_int(a);
  int best = 0;
  if (a > 0) {
    const bool cand = acc == a;
    if (!typical) {
      const uint64_t m = __ballot(cand);
      best = __ffsll((unsigned long long)m) - 1;
    } else {
      float l = cand ? lik : -INFINITY;
      l = wave_max(l);
      const uint64_t m = __ballot(cand && lik == l);
      best = __ffsll((unsigned long long)m) - 1;
    }
  } else {
    a = 0;
  }
  if (p == 0) {
    const int sel = t->retrieve[best * MEDUSA_MAX_TREE + a];
    best_out[b] = best;
    acc_out[b] = a;
    sel_out[b] = sel;
    root_out[b] = s[sel].amax;
  }
}

}  // namespace

extern "C" size_t evaluate_posterior_workspace_size(int B, int T) {
  if (B <= 0 || T <= 0) return 0;
  return align_up((size_t)B * T * sizeof(NodeStat), 256);
}

extern "C" int evaluate_posterior(const medusa_tree* t, int B, int V, const float* logits, const int32_t* tree_tokens,
                                  int mode, float temperature, float eps, float delta, int32_t* best,
                                  int32_t* accept_len, int32_t* sel_node, int32_t* next_root, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  MEDUSA_REQUIRE(B >= 0 && V > 0, MEDUSA_ERR_ARG, "evaluate_posterior: bad sizes");
  MEDUSA_REQUIRE(mode == MEDUSA_GREEDY || mode == MEDUSA_TYPICAL, MEDUSA_ERR_ARG, "evaluate_posterior: mode %d",
                 mode);
  MEDUSA_REQUIRE(mode == MEDUSA_GREEDY || temperature > 0.f, MEDUSA_ERR_ARG,
                 "evaluate_posterior: typical acceptance needs temperature > 0");
  MEDUSA_REQUIRE(t, MEDUSA_ERR_ARG, "evaluate_posterior: null tree");
  MEDUSA_REQUIRE(t->host.P <= 64, MEDUSA_ERR_UNSUPPORTED, "evaluate_posterior: more than 64 paths");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(logits && tree_tokens && best && accept_len && sel_node && next_root, MEDUSA_ERR_ARG,
                 "evaluate_posterior: null pointer");
  const int T = t->host.T;
  MEDUSA_REQUIRE(ws && ws_bytes >= evaluate_posterior_workspace_size(B, T), MEDUSA_ERR_WORKSPACE,
                 "evaluate_posterior: workspace %zu < %zu", ws_bytes, evaluate_posterior_workspace_size(B, T));
  NodeStat* st = (NodeStat*)ws;
  const int typical = mode == MEDUSA_TYPICAL;
  const float inv_tau = typical ? 1.0f / temperature : 1.0f;
  const int vec = V % 4 == 0 && ((uintptr_t)logits & 15) == 0;
  const int nv = vec ? (V / 4 + kStatThreads - 1) / kStatThreads : 0;
#define NS_LAUNCH(NVV)                                                                                        \
  hipLaunchKernelGGL(node_stats_kernel<NVV>, dim3(T, B), dim3(kStatThreads), 0, stream, logits, T, V, vec,  \
                     typical, inv_tau, eps, delta, st)
  if (nv == 1) NS_LAUNCH(1);
  else if (nv == 2) NS_LAUNCH(2);
  else if (nv == 3 || nv == 4) NS_LAUNCH(4);
  else if (nv >= 5 && nv <= 8) NS_LAUNCH(8);
  else NS_LAUNCH(0);  // unaligned rows, or rows past 8 * 4 * kStatThreads entries
#undef NS_LAUNCH
  int rc = check_launch("evaluate_posterior stats");
  if (rc) return rc;
  hipLaunchKernelGGL(select_kernel, dim3(B), dim3(64), 0, stream, t->dev, logits, V, tree_tokens, typical, inv_tau,
                     st, best, accept_len, sel_node, next_root);
  return check_launch("evaluate_posterior select");
}
