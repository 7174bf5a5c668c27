// Sampled tokens: the root under sampling = 'typical' / 'nucleus' and the draws
// of the non-fast acceptance branch.
//
// Page "大模型推理 memory bandwidth bound (5) - Medusa": generate_candidates()
// (section 二.4) draws the root from the last logits unless the temperature is 0
// or `fast` is set -- get_typical_one_token / get_nucleus_one_token (top_p 0.8 by
// default, section 二.1); section 一.3 defines the typical allow set
// {x : p(x) > min(eps, delta exp(-H))}; evaluate_posterior() (section 二.6)
// outside the fast branch keeps the first path of the longest accepted length.
// The bodies of those functions are not on the page; the readings taken:
//   q = softmax(logits / temperature); typical keeps {q > eta} (eta as in the
//   acceptance rule, entropy with the 1e-5 inside the log; an empty set leaves
//   the argmax); nucleus keeps the smallest set of the most probable tokens
//   whose mass reaches top_p, every token tied with the last one included;
//   the draw is the allowed token with the largest log q(x) + G(x),
//   G = -log(-log U) (Gumbel-max), lowest index on ties, U from Philox4x32-10
//   (Salmon, Moraes, Dror, Shaw, SC 2011) keyed by the 64-bit seed with counter
//   (x / 4, position, sequence, 0), output word x % 4, U = (2 (r >> 9) + 1) / 2^24;
//   non-fast acceptance draws at every tree node (its own position) and accepts
//   a candidate equal to the draw at its parent; the next root is the draw at
//   the selected node.
//
// One 1024-thread block per row: pass 1 finds the argmax, the maximum m and
// Z = sum 2^((x - m) log2(e) / tau); typical adds the entropy pass; nucleus
// bisects the probability threshold over the float bit patterns (31 passes of
// the mass at or above a candidate threshold, from L2); a last pass generates
// the uniforms and keeps the best allowed score.  Rows are read with float4
// loads when V % 4 == 0 and the rows are 16-byte aligned, and held in registers
// when V <= 32768.
#include "common.h"
#include "medusa_model.h"
#include "tree_dev.h"

using namespace medusa;

namespace {

constexpr int kDrawThreads = 1024;
constexpr int kDrawWaves = kDrawThreads / 64;

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

__device__ __forceinline__ float u01(uint32_t r) { return (float)(2u * (r >> 9) + 1u) * (1.0f / 16777216.0f); }

__device__ __forceinline__ bool score_better(float s, int i, float s2, int i2) {
  return s > s2 || (s == s2 && i < i2);
}

// block-wide sum (fixed order: lanes by xor steps, then waves in index order)
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kDrawWaves; ++j) s += red[j];
  return s;
}

struct DrawArgs {
  const float* logits;
  int64_t ld;
  int V;
  int vec;             // rows read as float4: V % 4 == 0, ld % 4 == 0, 16-byte aligned base
  const int32_t* seq;  // nullable: the sequence of row r is r / rows_per_seq
  int rows_per_seq;
  const int32_t* pos;
  int kind;
  float inv_tau, eps, delta, top_p;
  uint32_t k0, k1;
  int32_t* out;
};

// NV > 0 (float4 rows of at most NV * 4 * kDrawThreads entries): the row and its
// probabilities q are held in registers, NV float4 a thread, loaded once; the
// entropy pass, the nucleus bisection and the draw then read no memory.  NV == 0
// reads the row from memory in every pass (from L2 after the first).  Each
// thread visits its entries in the same order either way (thread tid owns float4
// tid, tid + kDrawThreads, ...) and q is the same function of the logit, so the
// draws are the same.
template <int NV>
__global__ __launch_bounds__(kDrawThreads) void draw_kernel(DrawArgs a) {
  const int row = blockIdx.x;
  const float* x = a.logits + (size_t)row * a.ld;
  const int V = a.V, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool vec = NV > 0 || a.vec;
  const int V4 = V / 4;
  __shared__ float s_v[kDrawWaves], s_f[kDrawWaves];
  __shared__ int s_i[kDrawWaves];
  __shared__ float red[kDrawWaves];
  const float c2 = a.inv_tau * 1.4426950408889634f;
  float4 f[NV > 0 ? NV : 1];
  if constexpr (NV > 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int k4 = tid + i * kDrawThreads;
      f[i] = ((const float4*)x)[k4 < V4 ? k4 : V4 - 1];  // a clamped index: the loads go out together
    }
  }
  // fn(v, k4) on each float4 of this thread's stripe, in stripe order (vec rows)
  auto each4 = [&](auto&& fn) __attribute__((always_inline)) {
    if constexpr (NV > 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int k4 = tid + i * kDrawThreads;
        if (k4 < V4) fn(f[i], k4, i);
      }
    } else {
      for (int k4 = tid; k4 < V4; k4 += kDrawThreads) fn(((const float4*)x)[k4], k4, 0);
    }
  };

  // ---- pass 1: argmax (lowest index on ties), max, Z
  float bv = -INFINITY, z = 0.f;
  int bi = 0x7fffffff;
  auto visit = [&](float v, int k) {
    if (v > bv) {
      z = z * __builtin_amdgcn_exp2f((bv - v) * c2) + 1.0f;
      bv = v;
      bi = k;
    } else {
      z += __builtin_amdgcn_exp2f((v - bv) * c2);
    }
  };
  if (vec) {
    each4([&](float4 g, int k4, int) {
      visit(g.x, 4 * k4);
      visit(g.y, 4 * k4 + 1);
      visit(g.z, 4 * k4 + 2);
      visit(g.w, 4 * k4 + 3);
    });
  } else {
    for (int k = tid; k < V; k += kDrawThreads) visit(x[k], k);
  }
  auto merge = [&](float v2, int i2, float z2) {
    const float m = fmaxf(bv, v2);
    if (m != -INFINITY) z = z * __builtin_amdgcn_exp2f((bv - m) * c2) + z2 * __builtin_amdgcn_exp2f((v2 - m) * c2);
    if (v2 > bv || (v2 == bv && i2 < bi)) {
      bv = v2;
      bi = i2;
    }
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
    for (int j = 1; j < kDrawWaves; ++j) merge(s_v[j], s_i[j], s_f[j]);
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
  if (bi == 0x7fffffff) bi = 0;
  const float m = bv, invZ = 1.0f / z;
  auto qof = [&](float v) { return __builtin_amdgcn_exp2f((v - m) * c2) * invZ; };
  // q of the held entries (NV > 0), computed once
  float4 qh[NV > 0 ? NV : 1];
  if constexpr (NV > 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) qh[i] = make_float4(qof(f[i].x), qof(f[i].y), qof(f[i].z), qof(f[i].w));
  }
  auto q4 = [&](float4 g, int i) __attribute__((always_inline)) {
    if constexpr (NV > 0) return qh[i];
    else return make_float4(qof(g.x), qof(g.y), qof(g.z), qof(g.w));
  };

  // ---- the allow set: q > eta (typical) or q >= t (nucleus)
  float thr = 0.f;
  bool strict = true;
  if (a.kind == MEDUSA_SAMPLE_TYPICAL) {
    float hs = 0.f;
    if (vec) {
      each4([&](float4 g, int, int i) {
        const float4 q = q4(g, i);
        hs += q.x * __builtin_amdgcn_logf(q.x + 1e-5f) + q.y * __builtin_amdgcn_logf(q.y + 1e-5f) +
              q.z * __builtin_amdgcn_logf(q.z + 1e-5f) + q.w * __builtin_amdgcn_logf(q.w + 1e-5f);
      });
    } else {
      for (int k = tid; k < V; k += kDrawThreads) {
        const float q = qof(x[k]);
        hs += q * __builtin_amdgcn_logf(q + 1e-5f);
      }
    }
    // base-2 logarithm above: the entropy in nats is -ln2 * sum
    const float H = -block_sum(hs, red) * 0.6931471805599453f;
    thr = fminf(a.eps, a.delta * expf(-H));
  } else {
    // largest t with mass(q >= t) >= top_p, by bisection over the bit patterns of
    // non-negative floats (ordered like their values); q(argmax) = 1/Z is the largest q
    uint32_t lo = 0u, hi = __float_as_uint(invZ) + 1u;  // mass(lo) = 1 >= top_p > mass(hi) = 0
    if (!(a.top_p > 0.f)) lo = __float_as_uint(invZ);
    while (hi - lo > 1u) {
      const uint32_t mid = lo + (hi - lo) / 2u;
      const float t = __uint_as_float(mid);
      float s = 0.f;
      if (vec) {
        each4([&](float4 g, int, int i) {
          const float4 q = q4(g, i);
          s += (q.x >= t ? q.x : 0.f) + (q.y >= t ? q.y : 0.f) + (q.z >= t ? q.z : 0.f) + (q.w >= t ? q.w : 0.f);
        });
      } else {
        for (int k = tid; k < V; k += kDrawThreads) {
          const float q = qof(x[k]);
          s += q >= t ? q : 0.f;
        }
      }
      if (block_sum(s, red) >= a.top_p)
        lo = mid;
      else
        hi = mid;
    }
    thr = __uint_as_float(lo);
    strict = false;
  }

  // ---- Gumbel-max over the allowed tokens
  const int seq = a.seq ? a.seq[row] : row / a.rows_per_seq;
  const uint32_t p = (uint32_t)a.pos[row];
  float bs = -INFINITY;
  int bt = 0x7fffffff;
  auto take = [&](float v, float q, int k, uint32_t r) {
    const bool ok = strict ? q > thr : q >= thr;
    if (!ok) return;
    const float s = (v - m) * a.inv_tau - logf(-logf(u01(r)));
    if (score_better(s, k, bs, bt)) {
      bs = s;
      bt = k;
    }
  };
  if (vec) {
    each4([&](float4 g, int j, int i) {
      const uint4 r = philox4x32_10(make_uint4((uint32_t)j, p, (uint32_t)seq, 0u), a.k0, a.k1);
      const float4 q = q4(g, i);
      const int k = 4 * j;
      take(g.x, q.x, k, r.x);
      take(g.y, q.y, k + 1, r.y);
      take(g.z, q.z, k + 2, r.z);
      take(g.w, q.w, k + 3, r.w);
    });
  } else {
    for (int j = tid; j < (V + 3) / 4; j += kDrawThreads) {
      const uint4 r = philox4x32_10(make_uint4((uint32_t)j, p, (uint32_t)seq, 0u), a.k0, a.k1);
      const int k = 4 * j;
      if (k < V) take(x[k], qof(x[k]), k, r.x);
      if (k + 1 < V) take(x[k + 1], qof(x[k + 1]), k + 1, r.y);
      if (k + 2 < V) take(x[k + 2], qof(x[k + 2]), k + 2, r.z);
      if (k + 3 < V) take(x[k + 3], qof(x[k + 3]), k + 3, r.w);
    }
  }
  butterfly([&](auto S) {
    constexpr int s = decltype(S)::value;
    const float s2 = bfly<s>(bs);
    const int t2 = bfly<s>(bt);
    if (score_better(s2, t2, bs, bt)) {
      bs = s2;
      bt = t2;
    }
  });
  __syncthreads();
  if (lane == 0) {
    s_v[w] = bs;
    s_i[w] = bt;
  }
  __syncthreads();
  if (tid == 0) {
    bs = s_v[0];
    bt = s_i[0];
    for (int j = 1; j < kDrawWaves; ++j)
      if (score_better(s_v[j], s_i[j], bs, bt)) {
        bs = s_v[j];
        bt = s_i[j];
      }
    a.out[row] = bt == 0x7fffffff ? bi : bt;  // nothing allowed: the argmax
  }
}

// grid rows x kDrawThreads: the register-held row when it fits
void launch_draw(unsigned rows, hipStream_t stream, const DrawArgs& a) {
  const int nv = a.vec ? (a.V / 4 + kDrawThreads - 1) / kDrawThreads : 0;
  if (nv == 1) hipLaunchKernelGGL(draw_kernel<1>, dim3(rows), dim3(kDrawThreads), 0, stream, a);
  else if (nv == 2) hipLaunchKernelGGL(draw_kernel<2>, dim3(rows), dim3(kDrawThreads), 0, stream, a);
  else if (nv == 3 || nv == 4) hipLaunchKernelGGL(draw_kernel<4>, dim3(rows), dim3(kDrawThreads), 0, stream, a);
  else if (nv >= 5 && nv <= 8) hipLaunchKernelGGL(draw_kernel<8>, dim3(rows), dim3(kDrawThreads), 0, stream, a);
  else hipLaunchKernelGGL(draw_kernel<0>, dim3(rows), dim3(kDrawThreads), 0, stream, a);
}

// One wave per sequence, lane p = path p: leading candidates equal to the draw at
// their parent; the first path of the longest accepted length; the next root is
// the draw at the selected node.
__global__ __launch_bounds__(64) void select_match_kernel(const medusa_tree_host* __restrict__ t,
                                                          const int32_t* __restrict__ tree_tokens,
                                                          const int32_t* __restrict__ draws, int32_t* __restrict__ best_out,
                                                          int32_t* __restrict__ acc_out, int32_t* __restrict__ sel_out,
                                                          int32_t* __restrict__ root_out) {
  const int b = blockIdx.x, p = threadIdx.x;
  const int T = t->T, P = t->P;
  const int32_t* d = draws + (size_t)b * T;
  int acc = -1;
  if (p < P) {
    acc = 0;
    const int len = t->path_len[p];
    const int32_t* rowp = t->retrieve + p * MEDUSA_MAX_TREE;
    for (int j = 1; j < len; ++j) {
      if (tree_tokens[(size_t)b * T + rowp[j]] != d[rowp[j - 1]]) break;
      ++acc;
    }
  }
  int amax = acc;
  amax = wave_max_int(amax);
  int best = 0;
  if (amax > 0) {
    const uint64_t msk = __ballot(acc == amax);
    best = __ffsll((unsigned long long)msk) - 1;
  } else {
    amax = 0;
  }
  if (p == 0) {
    const int sel = t->retrieve[best * MEDUSA_MAX_TREE + amax];
    best_out[b] = best;
    acc_out[b] = amax;
    sel_out[b] = sel;
    root_out[b] = d[sel];
  }
}

int check_sampling(const medusa_sampling* s) {
  MEDUSA_REQUIRE(s, MEDUSA_ERR_ARG, "sampling: null parameters");
  MEDUSA_REQUIRE(s->kind == MEDUSA_SAMPLE_TYPICAL || s->kind == MEDUSA_SAMPLE_NUCLEUS, MEDUSA_ERR_ARG,
                 "sampling: kind %d", s->kind);
  MEDUSA_REQUIRE(s->temperature > 0.f, MEDUSA_ERR_ARG, "sampling: temperature must be > 0");
  return MEDUSA_OK;
}

DrawArgs draw_args(const medusa_sampling* s, const float* logits, int64_t ld, int V, const int32_t* seq,
                   int rows_per_seq, const int32_t* pos, int32_t* out) {
  DrawArgs a;
  a.logits = logits;
  a.ld = ld;
  a.V = V;
  a.vec = V % 4 == 0 && ld % 4 == 0 && ((uintptr_t)logits & 15) == 0;
  a.seq = seq;
  a.rows_per_seq = rows_per_seq;
  a.pos = pos;
  a.kind = s->kind;
  a.inv_tau = 1.0f / s->temperature;
  a.eps = s->eps;
  a.delta = s->delta;
  a.top_p = s->top_p;
  a.k0 = (uint32_t)(s->seed & 0xffffffffull);
  a.k1 = (uint32_t)(s->seed >> 32);
  a.out = out;
  return a;
}

}  // namespace

extern "C" int medusa_sample_tokens(const medusa_sampling* s, int M, int V, const float* logits, int64_t ldx,
                                    const int32_t* seq_id, const int32_t* pos, int32_t* out, hipStream_t stream) {
  int rc = check_sampling(s);
  if (rc) return rc;
  MEDUSA_REQUIRE(M >= 0 && V > 0 && ldx >= V, MEDUSA_ERR_ARG, "sample_tokens: bad sizes");
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(logits && pos && out, MEDUSA_ERR_ARG, "sample_tokens: null pointer");
  launch_draw((unsigned)M, stream, draw_args(s, logits, ldx, V, seq_id, 1, pos, out));
  return check_launch("sample_tokens");
}

extern "C" size_t evaluate_posterior_sampled_workspace_size(int B, int T) {
  if (B <= 0 || T <= 0) return 0;
  return align_up((size_t)B * T * sizeof(int32_t), 256);
}

extern "C" int evaluate_posterior_sampled(const medusa_tree* t, int B, int V, const float* logits,
                                          const int32_t* tree_tokens, const int32_t* tree_pos,
                                          const medusa_sampling* s, int32_t* best, int32_t* accept_len,
                                          int32_t* sel_node, int32_t* next_root, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
  int rc = check_sampling(s);
  if (rc) return rc;
  MEDUSA_REQUIRE(B >= 0 && V > 0, MEDUSA_ERR_ARG, "evaluate_posterior_sampled: bad sizes");
  MEDUSA_REQUIRE(t, MEDUSA_ERR_ARG, "evaluate_posterior_sampled: null tree");
  MEDUSA_REQUIRE(t->host.P <= 64, MEDUSA_ERR_UNSUPPORTED, "evaluate_posterior_sampled: more than 64 paths");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(logits && tree_tokens && tree_pos && best && accept_len && sel_node && next_root, MEDUSA_ERR_ARG,
                 "evaluate_posterior_sampled: null pointer");
  const int T = t->host.T;
  MEDUSA_REQUIRE(ws && ws_bytes >= evaluate_posterior_sampled_workspace_size(B, T), MEDUSA_ERR_WORKSPACE,
                 "evaluate_posterior_sampled: workspace %zu < %zu", ws_bytes,
                 evaluate_posterior_sampled_workspace_size(B, T));
  int32_t* draws = (int32_t*)ws;
  launch_draw((unsigned)(B * T), stream, draw_args(s, logits, V, V, nullptr, T, tree_pos, draws));
  rc = check_launch("evaluate_posterior_sampled draws");
  if (rc) return rc;
  hipLaunchKernelGGL(select_match_kernel, dim3(B), dim3(64), 0, stream, t->dev, tree_tokens, draws, best, accept_len,
                     sel_node, next_root);
  return check_launch("evaluate_posterior_sampled select");
}
