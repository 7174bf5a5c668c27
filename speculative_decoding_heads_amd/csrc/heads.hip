// Medusa heads + per-head top-K.
//
// The page "大模型推理 memory bandwidth bound (5) - Medusa" defines a head as one
// residual block, p^(k) = softmax(W2^(k) (SiLU(W1^(k) h) + h)) (section 一.1),
// and generate_candidates() keeps the indices of each head's top-K logits
// (section 二.4; softmax is monotone, so the logits suffice).  The call runs
//   1. z = h + SiLU(W1 h) for all heads at once (W1 stacked [H*d, d]) with the
//      residual fused into the product's epilogue, z stored in the input dtype;
//   2. logits[b, k, :] = W2[k] z[b, k] as H batched products (fp32 out);
//   3. top-K per (b, k) row: for rows of at most 32768 entries, one
//      1024-thread workgroup per row (threshold from the thread maxima, the few
//      entries above it compacted in LDS, K selection rounds over them); for
//      longer rows in two stages: one wave per vocabulary chunk keeps a sorted per-lane
//      register list, then K rounds of a wave-wide (value desc, index asc)
//      maximum pop the chunk's K best; one wave per row merges the chunks'
//      candidates the same way.
#include <limits.h>
#include <stdlib.h>

#include "common.h"
#include "medusa_model.h"

using namespace medusa;

namespace {

constexpr int TK_MAX = 16;
constexpr int TK_PER_LANE = 8;  // vocabulary entries per lane in the first stage

__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Best (value desc, index asc) pair of a wave, in every lane, without LDS.  The
// pair travels as one 64-bit key whose unsigned order is the selection order
// (the value's bits made monotone above, the index complemented below), so each
// step is one 64-bit compare: DPP permutations inside each row of 16 lanes
// (swap neighbours, swap pairs, mirror within 8, mirror within 16), then the
// gfx950 row swaps (rows r and r ^ 1, then halves) -- each step pairs every lane
// with one not yet merged, and the maximum does not depend on the merge tree.
// -0 is keyed as +0 (the two tie, as under ==) and NaN below every number.
__device__ __forceinline__ uint64_t vi_key(float v, int i) {
  uint32_t u = __float_as_uint(v + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  u = v == v ? u : 0u;
  return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)i;
}
__device__ __forceinline__ void vi_unkey(uint64_t k, float& v, int& i) {
  const uint32_t u = (uint32_t)(k >> 32);
  v = __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
  i = (int)~(uint32_t)k;
}
template <int CTRL>
__device__ __forceinline__ uint64_t key_dpp(uint64_t k) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
  const uint64_t p = ((uint64_t)hi << 32) | lo;
  return p > k ? p : k;
}
// r[0], r[1] of a row swap with both operands the same register are the lane's
// own value and its partner's, in an order that is the same for both halves
template <int ROWS>
__device__ __forceinline__ uint64_t key_swap(uint64_t k) {
  const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
  const auto rl = ROWS == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                             : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto rh = ROWS == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                             : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const uint64_t a = ((uint64_t)rh[0] << 32) | rl[0], b = ((uint64_t)rh[1] << 32) | rl[1];
  return a > b ? a : b;
}
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  k = key_dpp<0xB1>(k);   // quad_perm [1,0,3,2]
  k = key_dpp<0x4E>(k);   // quad_perm [2,3,0,1]
  k = key_dpp<0x141>(k);  // row_half_mirror
  k = key_dpp<0x140>(k);  // row_mirror
  k = key_swap<16>(k);
  return key_swap<32>(k);
}
// (a -0 value comes back as +0)
__device__ __forceinline__ void wave_best(float& bv, int& bi) { vi_unkey(wave_max_key(vi_key(bv, bi)), bv, bi); }

// Per-lane sorted list (best first) of up to TK_MAX candidates.
struct LaneList {
  float v[TK_MAX];
  int i[TK_MAX];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int j = 0; j < TK_MAX; ++j) {
      v[j] = -INFINITY;
      i[j] = 0x7fffffff;
    }
  }
  __device__ __forceinline__ void insert(float x, int k) {
    if (!better(x, k, v[TK_MAX - 1], i[TK_MAX - 1])) return;
    v[TK_MAX - 1] = x;
    i[TK_MAX - 1] = k;
#pragma unroll
    for (int j = TK_MAX - 1; j > 0; --j) {
      if (better(v[j], i[j], v[j - 1], i[j - 1])) {
        const float tv = v[j];
        v[j] = v[j - 1];
        v[j - 1] = tv;
        const int ti = i[j];
        i[j] = i[j - 1];
        i[j - 1] = ti;
      }
    }
  }
  // K rounds of a wave-wide maximum; the owning lane pops its head each round.
  __device__ __forceinline__ void pop_k(int K, float* out_v, int* out_i) {
    for (int r = 0; r < K; ++r) {
      float bv = v[0];
      int bi = i[0];
      wave_best(bv, bi);
      if (threadIdx.x == 0) {
        out_v[r] = bv;
        out_i[r] = bi;
      }
      if (i[0] == bi && bi != 0x7fffffff) {
#pragma unroll
        for (int j = 0; j < TK_MAX - 1; ++j) {
          v[j] = v[j + 1];
          i[j] = i[j + 1];
        }
        v[TK_MAX - 1] = -INFINITY;
        i[TK_MAX - 1] = 0x7fffffff;
      }
    }
  }
};

// stage 1: grid (n_chunks, M), one wave per chunk of a row -> K candidates per
// chunk, in two passes over the chunk.  Pass 1 takes each lane's maximum; the
// K-th largest of the 64 lane maxima, t, is a lower bound of the chunk's K-th
// largest value (K lanes each hold an entry >= t).  Pass 2 (the chunk is now in
// L2) inserts only the entries >= t into the lane lists, so the sorted-list
// insertion, which a wave executes whenever any of its lanes needs it, runs
// for a few entries per chunk instead of for most of them.  With vec (rows
// 16-byte aligned, chunk % 256 == 0) lanes read float4 batches, 8 per lane in
// flight together.
__global__ __launch_bounds__(64) void topk_stage1_kernel(int V, int chunk, const float* __restrict__ x, int K,
                                                         float* __restrict__ cv, int* __restrict__ ci, int vec) {
  const int ch = blockIdx.x, row = blockIdx.y, nch = gridDim.x;
  const float* r = x + (size_t)row * V;
  const int k0 = ch * chunk, k1 = min(k0 + chunk, V);
  const int lane = threadIdx.x;
  constexpr int BATCH = 8 * 4 * 64;  // entries per wave and float4 batch
  // visit every entry of the chunk: batches of float4, then a scalar tail
  auto scan = [&](auto&& f) __attribute__((always_inline)) {
    int k = k0;
    if (vec) {
      for (; k + BATCH <= k1; k += BATCH) {
        float4 b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) b[u] = *(const float4*)(r + k + 256 * u + 4 * lane);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int kb = k + 256 * u + 4 * lane;
          f(b[u].x, kb);
          f(b[u].y, kb + 1);
          f(b[u].z, kb + 2);
          f(b[u].w, kb + 3);
        }
      }
    }
    for (k += lane; k < k1; k += 64) f(r[k], k);
  };
  float lm = -INFINITY;
  scan([&](float v, int) __attribute__((always_inline)) { lm = fmaxf(lm, v); });
  // K-th largest lane maximum (each round removes the largest, lowest lane first)
  float t = -INFINITY;
  {
    float v = lm;
    for (int rd = 0; rd < K; ++rd) {
      float bv = v;
      int bl = lane;
      wave_best(bv, bl);
      t = bv;
      if (lane == bl) v = -INFINITY;
    }
  }
  LaneList L;
  L.init();
  scan([&](float v, int k) __attribute__((always_inline)) {
    if (v >= t) L.insert(v, k);
  });
  const size_t o = ((size_t)row * nch + ch) * K;
  L.pop_k(K, cv + o, ci + o);
}

// stage 2: grid (M), one wave merges n_chunks * K candidates
__global__ __launch_bounds__(64) void topk_stage2_kernel(int ncand, const float* __restrict__ cv,
                                                         const int* __restrict__ ci, int K, int32_t* __restrict__ idx,
                                                         float* __restrict__ val) {
  const int row = blockIdx.x;
  LaneList L;
  L.init();
  for (int j = threadIdx.x; j < ncand; j += 64) L.insert(cv[(size_t)row * ncand + j], ci[(size_t)row * ncand + j]);
  __shared__ float sv[TK_MAX];
  __shared__ int si[TK_MAX];
  L.pop_k(K, sv, si);
  __syncthreads();
  if ((int)threadIdx.x < K) {
    const int t = si[threadIdx.x];
    idx[(size_t)row * K + threadIdx.x] = t == 0x7fffffff ? 0 : t;
    if (val) val[(size_t)row * K + threadIdx.x] = sv[threadIdx.x];
  }
}

// One workgroup of 1024 threads per row (rows of at most 8 * 4096 entries):
// the whole row sits in registers (NV float4 batches a thread) and the top K
// come out of three steps with no second launch.
//  1. t = the K-th largest of the 1024 thread maxima: they go to LDS and one
//     wave takes K rounds of a wave maximum over them (16 a lane), while the
//     other waves wait at the barrier (sixteen waves ranking the same values
//     would share the four SIMDs and each run four times slower).  The K
//     threads behind those maxima hold K distinct entries >= t, so the row's
//     K-th largest entry is >= t.
//  2. Every entry >= t is appended to an LDS list (typically a few dozen).
//  3. One wave takes K rounds of a (value desc, index asc) maximum over the
//     list: with at most 64 entries each lane holds one as a 64-bit key
//     (vi_key) and the winner of a round drops out; with more, each round
//     re-reads the list and keeps the entries strictly after the previous
//     winner.
// If more than TR_CAP entries reach t (a plateau of equal values), step 3 runs
// over every thread's registers instead, with a block-wide maximum per round.
// Either way the result is the exact top K in that order.
constexpr int TR_THREADS = 1024;
constexpr int TR_WAVES = TR_THREADS / 64;
constexpr int TR_CAP = 2048;
constexpr int TR_MAX_NV = 8;  // rows up to 8 * 4 * 1024 = 32768 entries (longer rows spill registers)

template <int NV>
__global__ __launch_bounds__(TR_THREADS) void topk_row_kernel(int V, const float* __restrict__ x, int K, int vec,
                                                              int32_t* __restrict__ idx, float* __restrict__ val) {
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* r = x + (size_t)row * V;
  __shared__ float s_tm[TR_THREADS];
  __shared__ float s_t;
  __shared__ float s_cv[TR_CAP];
  __shared__ int s_ci[TR_CAP];
  __shared__ float s_rv[2][TR_WAVES];
  __shared__ int s_ri[2][TR_WAVES];
  __shared__ int s_cnt;
  // element e = 4u + c of this thread: index (u * 1024 + tid) * 4 + c (float4
  // batches) or (4u + c) * 1024 + tid (scalar loads)
  auto index_of = [&](int u, int c) __attribute__((always_inline)) {
    return vec ? (u * TR_THREADS + tid) * 4 + c : (4 * u + c) * TR_THREADS + tid;
  };
  float v[NV * 4];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    if (vec && (u * TR_THREADS + tid) * 4 + 3 < V) {
      const float4 b = *(const float4*)(r + (u * TR_THREADS + tid) * 4);
      v[4 * u] = b.x;
      v[4 * u + 1] = b.y;
      v[4 * u + 2] = b.z;
      v[4 * u + 3] = b.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int k = index_of(u, c);
        v[4 * u + c] = k < V ? r[k] : -INFINITY;
      }
    }
  }
  if (tid == 0) s_cnt = 0;
  // 1. threshold
  float tm = -INFINITY;
#pragma unroll
  for (int e = 0; e < NV * 4; ++e) tm = fmaxf(tm, v[e]);
  s_tm[tid] = tm;
  __syncthreads();
  if (w == 0) {
    // lane holds the maxima of threads lane + 64 q; lb = the best of them left
    uint64_t lk[TR_WAVES];
#pragma unroll
    for (int q = 0; q < TR_WAVES; ++q) lk[q] = vi_key(s_tm[lane + 64 * q], lane + 64 * q);
    auto lane_best = [&]() __attribute__((always_inline)) {
      uint64_t b = lk[0];
#pragma unroll
      for (int q = 1; q < TR_WAVES; ++q) b = lk[q] > b ? lk[q] : b;
      return b;
    };
    uint64_t lb = lane_best(), km = 0;
    for (int rd = 0; rd < K; ++rd) {
      km = wave_max_key(lb);
      if (km == lb) {  // the winning thread's lane (keys are distinct) drops it
        const int wq = (int)~(uint32_t)km >> 6;
#pragma unroll
        for (int q = 0; q < TR_WAVES; ++q) lk[q] = q == wq ? 0 : lk[q];
        lb = lane_best();
      }
    }
    if (lane == 0) {
      float tv;
      int ti;
      vi_unkey(km, tv, ti);
      s_t = tv;
    }
  }
  __syncthreads();
  const float t = s_t;
  // 2. entries >= t into the LDS list
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = index_of(u, c);
      if (k < V && v[4 * u + c] >= t) {
        const int p = atomicAdd(&s_cnt, 1);
        if (p < TR_CAP) {
          s_cv[p] = v[4 * u + c];
          s_ci[p] = k;
        }
      }
    }
  __syncthreads();
  const int n = s_cnt;
  // 3. K rounds of a maximum over the list
  if (n <= 64) {
    if (w != 0) return;
    const float cv = lane < n ? s_cv[lane] : -INFINITY;
    const int ci = lane < n ? s_ci[lane] : 0;
    uint64_t k = lane < n ? vi_key(cv, ci) : 0;
    for (int rd = 0; rd < K; ++rd) {
      const uint64_t km = wave_max_key(k);
      if (km != 0 && k == km) {  // the winner writes its own entry and drops out
        idx[(size_t)row * K + rd] = ci;
        if (val) val[(size_t)row * K + rd] = cv;
        k = 0;
      } else if (km == 0 && lane == 0) {  // fewer than K entries (rows of NaN)
        idx[(size_t)row * K + rd] = 0;
        if (val) val[(size_t)row * K + rd] = -INFINITY;
      }
    }
    return;
  }
  // ... each round over the entries strictly after the previous winner
  float pv = INFINITY;
  int pi = -1;
  if (n <= TR_CAP) {
    if (w != 0) return;
    for (int rd = 0; rd < K; ++rd) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int j = lane; j < n; j += 64) {
        const float cv = s_cv[j];
        const int ci = s_ci[j];
        if (better(pv, pi, cv, ci) && better(cv, ci, bv, bi)) {
          bv = cv;
          bi = ci;
        }
      }
      wave_best(bv, bi);
      if (lane == 0) {
        idx[(size_t)row * K + rd] = bi == 0x7fffffff ? 0 : bi;
        if (val) val[(size_t)row * K + rd] = bv;
      }
      pv = bv;
      pi = bi;
    }
    return;
  }
  for (int rd = 0; rd < K; ++rd) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < NV; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int k = index_of(u, c);
        const float cv = v[4 * u + c];
        if (k < V && better(pv, pi, cv, k) && better(cv, k, bv, bi)) {
          bv = cv;
          bi = k;
        }
      }
    wave_best(bv, bi);
    if (lane == 0) {
      s_rv[rd & 1][w] = bv;
      s_ri[rd & 1][w] = bi;
    }
    __syncthreads();
    bv = s_rv[rd & 1][0];
    bi = s_ri[rd & 1][0];
    for (int j = 1; j < TR_WAVES; ++j)
      if (better(s_rv[rd & 1][j], s_ri[rd & 1][j], bv, bi)) {
        bv = s_rv[rd & 1][j];
        bi = s_ri[rd & 1][j];
      }
    if (tid == 0) {
      idx[(size_t)row * K + rd] = bi == 0x7fffffff ? 0 : bi;
      if (val) val[(size_t)row * K + rd] = bv;
    }
    pv = bv;
    pi = bi;
  }
}

// Chunks per row: 512-entry chunks (TK_PER_LANE entries per lane) while the
// rows are few; with many rows fewer, longer chunks (about 4096 waves in all),
// so that each wave's fixed cost of handing on K candidates is spread over more
// entries.
int topk_chunks(int M, int V) {
  const int nmax = (V + 64 * TK_PER_LANE - 1) / (64 * TK_PER_LANE);
  int n = (4096 + M - 1) / M;
  if (n > nmax) n = nmax;
  return n < 1 ? 1 : (n > 1024 ? 1024 : n);
}

size_t topk_ws(int M, int V, int K) {
  return align_up((size_t)M * topk_chunks(M, V) * K * (sizeof(float) + sizeof(int)), 256);
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
  size_t g3 = topk_ws(B * H, V, TK_MAX);
  size_t g = g1 > g2 ? g1 : g2;
  L.total = L.gemm_off + (g > g3 ? g : g3);
  return L;
}

}  // namespace

extern "C" size_t medusa_topk_rows_workspace_size(int M, int V, int K) {
  if (M <= 0 || V <= 0 || K <= 0) return 0;
  return topk_ws(M, V, K);
}

extern "C" int medusa_topk_rows(int M, int V, const float* x, int K, int32_t* idx, float* val, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  MEDUSA_REQUIRE(M >= 0 && V > 0, MEDUSA_ERR_ARG, "topk_rows: bad sizes");
  MEDUSA_REQUIRE(K >= 1 && K <= TK_MAX && K <= V, MEDUSA_ERR_UNSUPPORTED, "topk_rows: K=%d not in [1, %d]", K, TK_MAX);
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(x && idx, MEDUSA_ERR_ARG, "topk_rows: null pointer");
  MEDUSA_REQUIRE(ws && ws_bytes >= topk_ws(M, V, K), MEDUSA_ERR_WORKSPACE, "topk_rows: workspace %zu < %zu", ws_bytes,
                 topk_ws(M, V, K));
  const int vec4 = V % 4 == 0 && ((uintptr_t)x & 15) == 0;
  const int nv = (V + 4 * TR_THREADS - 1) / (4 * TR_THREADS);
  // One workgroup per row for rows of at most 32768 entries: measured at V 32000
  // and K 10 against the two-stage path (each row spread over many waves),
  // 11 vs 26 us at 4 rows, 25 vs 47 us at 512, 51 vs 63 us at 1024 and 96 vs
  // 108 us at 2048.  MEDUSA_TOPK_ROW_MAX_M sends larger row counts to the
  // two-stage path (tuning runs).
  static const int e_rows = [] {
    const char* e = getenv("MEDUSA_TOPK_ROW_MAX_M");
    return e ? atoi(e) : INT_MAX;
  }();
  if (nv <= TR_MAX_NV && M <= e_rows) {
#define TR_LAUNCH(NVV) \
  hipLaunchKernelGGL(topk_row_kernel<NVV>, dim3(M), dim3(TR_THREADS), 0, stream, V, x, K, vec4, idx, val)
    if (nv <= 1) TR_LAUNCH(1);
    else if (nv <= 2) TR_LAUNCH(2);
    else if (nv <= 4) TR_LAUNCH(4);
    else TR_LAUNCH(8);
#undef TR_LAUNCH
    return check_launch("topk_rows");
  }
  const int nch = topk_chunks(M, V);
  int chunk = (V + nch - 1) / nch;
  const int vec = V % 4 == 0 && ((uintptr_t)x & 15) == 0;
  if (vec) chunk = (chunk + 255) / 256 * 256;  // batches start 16-byte aligned
  float* cv = (float*)ws;
  int* ci = (int*)((char*)ws + (size_t)M * nch * K * sizeof(float));
  hipLaunchKernelGGL(topk_stage1_kernel, dim3(nch, M), dim3(64), 0, stream, V, chunk, x, K, cv, ci, vec);
  int rc = check_launch("topk_rows stage 1");
  if (rc) return rc;
  hipLaunchKernelGGL(topk_stage2_kernel, dim3(M), dim3(64), 0, stream, nch * K, cv, ci, K, idx, val);
  return check_launch("topk_rows stage 2");
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
  return medusa_topk_rows(B * H, V, logits, K, topk_idx, topk_val, gws, gbytes, stream);
}
