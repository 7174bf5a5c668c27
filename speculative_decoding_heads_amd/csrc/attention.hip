// Tree attention: T tree queries against the KV prefix plus the tree's own KV
// under the ancestor-only mask.
//
// Semantics follow the page "大模型推理 memory bandwidth bound (5) - Medusa":
// section 一.2 (the candidate tree is flattened into one sequence; a node only
// attends to its predecessors on its own path), section 二.2 (the mask rows,
// root column all ones) and section 二.3 (the mask is installed on the base
// model, so every cached prefix token stays visible).  The mask arrives as one
// 64-bit word per node.
//
// Two kernels:
//  * attn_generic -- fp32 or bf16, any head size <= 128.  One wave per (query
//    node, query head).  Lane l owns the keys whose absolute sequence position
//    is l mod 64 (a tree node at depth d sits at position seq_len + d), walks
//    them in increasing position with an online softmax, and the 64 lane
//    states are merged in lane order.  The result therefore depends only on
//    the (position, key, value) triples a query sees, not on how they are split
//    between cache and tree: plain one-token decoding and tree verification of
//    the same accepted tokens give bit-identical outputs.
//  * attn_stream (attn_stream.hip) -- bf16, head size 64 or 128, the
//    streaming MFMA kernel; with KV splits it writes fp32 partials that
//    attn_combine (below) merges.
#include <math.h>
#include <stdlib.h>

#include <mutex>

#include "attn_stream.h"
#include "common.h"

using namespace medusa;

namespace {

// --------------------------------------------------------------------------
// generic kernel
// --------------------------------------------------------------------------
template <typename T, int DMAX>
__global__ __launch_bounds__(64) void attn_generic_kernel(const T* __restrict__ q, const T* __restrict__ Kc,
                                                          const T* __restrict__ Vc, int64_t Lmax,
                                                          const int32_t* __restrict__ seq_len,
                                                          const T* __restrict__ Kt, const T* __restrict__ Vt,
                                                          const uint64_t* __restrict__ anc, int Tn, int Hq, int Hkv,
                                                          int Dh, float scale, T* __restrict__ out) {
  const int i = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int G = Hq / Hkv;
  const int kvh = hq / G;
  __shared__ float s_q[DMAX];
  __shared__ float s_acc[64][DMAX + 1];
  __shared__ float s_m[64], s_l[64];
  const size_t qoff = (((size_t)b * Tn + i) * Hq + hq) * Dh;
  for (int d = lane; d < Dh; d += 64) s_q[d] = Elem<T>::load(q, qoff + d) * scale;
  __syncthreads();
  int64_t L = seq_len[b];
  if (L > Lmax) L = Lmax;
  if (L < 0) L = 0;
  float m = -INFINITY, l = 0.f;
  float acc[DMAX];
#pragma unroll
  for (int d = 0; d < DMAX; ++d) acc[d] = 0.f;

  auto visit = [&](const T* kr, const T* vr) {
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < DMAX; ++d)
      if (d < Dh) s += s_q[d] * Elem<T>::load(kr, d);
    const float mn = fmaxf(m, s);
    const float a = expf(m - mn);
    const float p = expf(s - mn);
    l = l * a + p;
#pragma unroll
    for (int d = 0; d < DMAX; ++d)
      if (d < Dh) acc[d] = acc[d] * a + p * Elem<T>::load(vr, d);
    m = mn;
  };

  const size_t slab = (size_t)b * Hkv + kvh;
  for (int64_t pos = lane; pos < L; pos += 64)
    visit(Kc + (slab * Lmax + pos) * Dh, Vc + (slab * Lmax + pos) * Dh);
  // tree keys: ancestors of i in increasing node index = increasing depth
  const uint64_t tmask = Tn >= 64 ? ~0ull : ((1ull << Tn) - 1ull);
  uint64_t bits = anc[i] & tmask;
  while (bits) {
    const int j = __ffsll((unsigned long long)bits) - 1;
    bits &= bits - 1;
    const int depth = __popcll(anc[j] & tmask) - 1;
    if ((int)((L + depth) & 63) == lane) visit(Kt + (slab * Tn + j) * Dh, Vt + (slab * Tn + j) * Dh);
  }
  s_m[lane] = m;
  s_l[lane] = l;
#pragma unroll
  for (int d = 0; d < DMAX; ++d)
    if (d < Dh) s_acc[lane][d] = acc[d];
  __syncthreads();
  float mt = -INFINITY;
  for (int j = 0; j < 64; ++j) mt = fmaxf(mt, s_m[j]);
  float lt = 0.f;
  for (int j = 0; j < 64; ++j) lt += s_l[j] * expf(s_m[j] - mt);
  const float inv = 1.0f / lt;
  for (int d = lane; d < Dh; d += 64) {
    float o = 0.f;
    for (int j = 0; j < 64; ++j) o += s_acc[j][d] * expf(s_m[j] - mt);
    Elem<T>::store(out, qoff + d, o * inv);
  }
}

constexpr int ATTN_MAX_SPLITS = 64;

// grid (ceil(R / 2), Hkv, B), block 64 threads: merge the split partials of
// two query rows, one half-wave a row, four dimensions a lane (16-byte
// loads).  Lane s of a half reads split s's maximum and sum (and s + 32's), the
// half-wave reduces them with cross-lane swaps, and each split's weight is
// then broadcast from its lane while the partial rows are added in split
// order.  Dh % 4 == 0, Dh <= 128, n_splits <= 64.
template <typename T>
__global__ __launch_bounds__(64) void attn_combine_kernel(const float* __restrict__ ws_o,
                                                          const float* __restrict__ ws_ml, int Tn, int Hq, int Hkv,
                                                          int Dh, int n_splits, T* __restrict__ out) {
  const int G = Hq / Hkv;
  const int R = Tn * G;
  const int lane = threadIdx.x & 31;
  const int r = blockIdx.x * 2 + (threadIdx.x >> 5);
  const bool valid = r < R;
  const int rr = valid ? r : R - 1;  // a half past the rows works on the last row and stores nothing
  const int kvh = blockIdx.y, b = blockIdx.z;
  const size_t slab = (size_t)b * Hkv + kvh;
  const size_t base = slab * n_splits * (size_t)R + rr;  // partial row of split s: base + s * R
  const int d0 = lane * 4 < Dh ? lane * 4 : 0;  // lanes past Dh load a valid column and store nothing
  // The first CB splits' partial rows do not depend on the weights: their
  // loads go out with the maximum/sum loads, so n_splits <= CB costs one
  // memory round trip (a split index past n_splits re-reads the last split
  // and is left out of the sum).
  constexpr int CB = 8;
  float4 v[CB];
#pragma unroll
  for (int u = 0; u < CB; ++u) {
    const int su = u < n_splits ? u : n_splits - 1;
    v[u] = *(const float4*)(ws_o + (base + (size_t)su * R) * Dh + d0);
  }
  float m0 = -INFINITY, l0 = 0.f, m1 = -INFINITY, l1 = 0.f;
  if (lane < n_splits) {
    m0 = ws_ml[(base + (size_t)lane * R) * 2];
    l0 = ws_ml[(base + (size_t)lane * R) * 2 + 1];
  }
  if (lane + 32 < n_splits) {
    m1 = ws_ml[(base + (size_t)(lane + 32) * R) * 2];
    l1 = ws_ml[(base + (size_t)(lane + 32) * R) * 2 + 1];
  }
  float mt = fmaxf(m0, m1);
  butterfly<5>([&](auto S) { mt = fmaxf(mt, bfly<decltype(S)::value>(mt)); });  // within the half wave
  const float w0 = m0 != -INFINITY ? __builtin_amdgcn_exp2f(m0 - mt) : 0.f;
  const float w1 = m1 != -INFINITY ? __builtin_amdgcn_exp2f(m1 - mt) : 0.f;
  float lt = l0 * w0 + l1 * w1;
  butterfly<5>([&](auto S) { lt += bfly<decltype(S)::value>(lt); });
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < CB; ++u) {
    const float w = __shfl(w0, u, 32);  // split u < 32: its weight sits in lane u's w0
    if (u < n_splits) {
      acc[0] += v[u].x * w;
      acc[1] += v[u].y * w;
      acc[2] += v[u].z * w;
      acc[3] += v[u].w * w;
    }
  }
  for (int s0 = CB; s0 < n_splits; s0 += CB) {
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int su = s0 + u < n_splits ? s0 + u : n_splits - 1;
      v[u] = *(const float4*)(ws_o + (base + (size_t)su * R) * Dh + d0);
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int s = s0 + u;
      const float w = __shfl(s < 32 ? w0 : w1, s & 31, 32);
      if (s < n_splits) {
        acc[0] += v[u].x * w;
        acc[1] += v[u].y * w;
        acc[2] += v[u].z * w;
        acc[3] += v[u].w * w;
      }
    }
  }
  if (!valid || lane * 4 >= Dh) return;
  const int node = r / G, g = r % G;
  const size_t ooff = (((size_t)b * Tn + node) * Hq + (size_t)kvh * G + g) * Dh;
#pragma unroll
  for (int i = 0; i < 4; ++i) Elem<T>::store(out, ooff + d0 + i, acc[i] * inv);
}

struct MfmaPlan {
  int nw, n_rchunks, n_splits;
  size_t ws_o_bytes, ws_ml_bytes;
};

MfmaPlan mfma_plan_nw(int B, int T, int Hq, int Hkv, int Dh, int64_t L_hint, int nw);

// Waves per workgroup and KV splits.  For each width nw in {8, 4, 2} the split
// count is the one that puts a workgroup on each of the 256 CUs, kept to at
// least 4 64-key tiles per split (mfma_plan_nw).  Among the widths whose plan
// fills the chip, the one whose splits run closest to 16 tiles (log scale;
// ties: more waves); if none fills, the one with the most workgroups (ties:
// more waves).  The two costs it trades: every split writes fp32 partials of
// all R query rows of its KV head (R x Dh x 4 bytes, at 4 tiles a split about
// what the split reads of K/V) that the merge reads back, and fewer waves mean
// more 32-row chunks, each streaming the same K/V again.  Measured on MI355X
// over batch 1, 2, 4 and 8, 8 and 32 KV heads x 128, prefixes 1k-64k and every
// (waves, splits) pair: within 0.5 % of the best pair summed over the 30
// cases, the worst 15-19 % off (batch 1 / prefix 8k and batch 2 / prefix 4k
// at 8 KV heads, where 4 waves and 8 tiles a split beat 2 waves and 16).  A
// cost model (tiles a split times a per-tile time by rows, plus the merge's
// partial bytes) ranks the same cases as well overall.  MEDUSA_ATTN_WAVES =
// 2 | 4 | 8 forces a width.
MfmaPlan mfma_plan(int B, int T, int Hq, int Hkv, int Dh, int64_t L_hint) {
  const int forced = attn_stream_waves_forced();
  if (forced) return mfma_plan_nw(B, T, Hq, Hkv, Dh, L_hint, forced);
  const int64_t tiles = (L_hint + ATTN_KT - 1) / ATTN_KT;
  MfmaPlan fill{}, most{};
  double fill_d = 0.0;
  int64_t most_wgs = -1;
  bool any_fill = false;
  for (int nw : {8, 4, 2}) {
    const MfmaPlan p = mfma_plan_nw(B, T, Hq, Hkv, Dh, L_hint, nw);
    const int64_t wgs = (int64_t)p.n_splits * Hkv * B * p.n_rchunks;
    if (wgs >= 256) {
      const int64_t tps = (tiles + p.n_splits - 1) / p.n_splits;
      const double d = fabs(log2((double)(tps > 0 ? tps : 1) / 16.0));
      if (!any_fill || d < fill_d) {
        fill = p;
        fill_d = d;
        any_fill = true;
      }
    }
    if (wgs > most_wgs) {
      most = p;
      most_wgs = wgs;
    }
  }
  return any_fill ? fill : most;
}

MfmaPlan mfma_plan_nw(int B, int T, int Hq, int Hkv, int Dh, int64_t L_hint, int nw) {
  MfmaPlan p;
  const int R = T * (Hq / Hkv);
  p.nw = nw;
  const int rows_wg = 32 * nw;
  p.n_rchunks = (R + rows_wg - 1) / rows_wg;
  const int64_t tiles = (L_hint + ATTN_KT - 1) / ATTN_KT;
  const int64_t units = (int64_t)B * Hkv * p.n_rchunks;
  // one workgroup per CU (256), each split at least min_tiles tiles
  // (MEDUSA_ATTN_MIN_TILES overrides the 4 for tuning runs)
  static const int min_tiles = [] {
    const char* e = getenv("MEDUSA_ATTN_MIN_TILES");
    const int v = e ? atoi(e) : 4;
    return v >= 1 ? v : 4;
  }();
  int64_t s = (256 + units - 1) / units;
  int64_t smax = tiles / min_tiles;
  if (smax > ATTN_MAX_SPLITS) smax = ATTN_MAX_SPLITS;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  p.n_splits = (int)s;
  if (p.n_splits > 1) {
    p.ws_o_bytes = align_up((size_t)B * Hkv * p.n_splits * R * Dh * sizeof(float), 256);
    p.ws_ml_bytes = align_up((size_t)B * Hkv * p.n_splits * R * 2 * sizeof(float), 256);
  } else {
    p.ws_o_bytes = p.ws_ml_bytes = 0;
  }
  return p;
}

bool use_mfma(int dtype, int Dh) { return dtype == MEDUSA_BF16 && (Dh == 64 || Dh == 128); }

}  // namespace

extern "C" size_t tree_attention_workspace_size(int dtype, int B, int T, int Hq, int Hkv, int Dh, int64_t L_hint) {
  if (B <= 0 || T <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !use_mfma(dtype, Dh)) return 0;
  MfmaPlan p = mfma_plan(B, T, Hq, Hkv, Dh, L_hint < 0 ? 0 : L_hint);
  return p.ws_o_bytes + p.ws_ml_bytes;
}

extern "C" int tree_attention(int dtype, int B, int T, int Hq, int Hkv, int Dh, const void* q, const void* Kc,
                              const void* Vc, int64_t Lmax, int64_t L_hint, const int32_t* seq_len, const void* Kt,
                              const void* Vt, const uint64_t* anc, float scale, void* out, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  MEDUSA_REQUIRE(dtype_ok(dtype), MEDUSA_ERR_UNSUPPORTED, "tree_attention: dtype %d", dtype);
  MEDUSA_REQUIRE(B >= 0 && T >= 1 && Hq >= 1 && Hkv >= 1 && Dh >= 1 && Lmax >= 0, MEDUSA_ERR_ARG,
                 "tree_attention: bad sizes");
  MEDUSA_REQUIRE(Hq % Hkv == 0, MEDUSA_ERR_ARG, "tree_attention: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  MEDUSA_REQUIRE(T <= MEDUSA_MAX_TREE, MEDUSA_ERR_UNSUPPORTED, "tree_attention: T=%d > %d", T, MEDUSA_MAX_TREE);
  MEDUSA_REQUIRE(L_hint >= 0 && L_hint <= Lmax, MEDUSA_ERR_ARG, "tree_attention: L_hint outside [0, Lmax]");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(q && Kt && Vt && anc && seq_len && out, MEDUSA_ERR_ARG, "tree_attention: null pointer");
  MEDUSA_REQUIRE(Lmax == 0 || (Kc && Vc), MEDUSA_ERR_ARG, "tree_attention: null cache pointer");
  if (use_mfma(dtype, Dh)) {
    MfmaPlan p = mfma_plan(B, T, Hq, Hkv, Dh, L_hint);
    MEDUSA_REQUIRE(p.ws_o_bytes + p.ws_ml_bytes <= ws_bytes && (p.n_splits == 1 || ws), MEDUSA_ERR_WORKSPACE,
                   "tree_attention: workspace %zu < %zu", ws_bytes, p.ws_o_bytes + p.ws_ml_bytes);
    float* ws_o = (float*)ws;
    float* ws_ml = p.n_splits > 1 ? (float*)((char*)ws + p.ws_o_bytes) : nullptr;
    const float sl2 = scale * 1.4426950408889634f;
    dim3 grid(p.n_splits, Hkv, B * p.n_rchunks);
    int rc = launch_attn_stream(Dh, p.nw, grid, stream, (const bf16_t*)q, (const bf16_t*)Kc, (const bf16_t*)Vc, Lmax, seq_len,
                                (const bf16_t*)Kt, (const bf16_t*)Vt, anc, T, Hq, Hkv, p.n_rchunks, sl2, p.n_splits,
                                (bf16_t*)out, ws_o, ws_ml);
    if (rc) return rc;
    if (p.n_splits > 1) {
      hipLaunchKernelGGL(attn_combine_kernel<bf16_t>, dim3((T * (Hq / Hkv) + 1) / 2, Hkv, B), dim3(64), 0, stream,
                         ws_o, ws_ml, T, Hq, Hkv, Dh, p.n_splits, (bf16_t*)out);
      return check_launch("tree_attention combine");
    }
    return MEDUSA_OK;
  }
  MEDUSA_REQUIRE(Dh <= 128, MEDUSA_ERR_UNSUPPORTED, "tree_attention: generic kernel takes Dh <= 128");
  dim3 grid(T, Hq, B);
#define GEN_LAUNCH(TY, DM)                                                                                     \
  hipLaunchKernelGGL((attn_generic_kernel<TY, DM>), grid, dim3(64), 0, stream, (const TY*)q, (const TY*)Kc,   \
                     (const TY*)Vc, Lmax, seq_len, (const TY*)Kt, (const TY*)Vt, anc, T, Hq, Hkv, Dh, scale, \
                     (TY*)out)
  if (dtype == MEDUSA_F32) {
    if (Dh <= 16) GEN_LAUNCH(float, 16);
    else if (Dh <= 32) GEN_LAUNCH(float, 32);
    else if (Dh <= 64) GEN_LAUNCH(float, 64);
    else GEN_LAUNCH(float, 128);
  } else {
    if (Dh <= 16) GEN_LAUNCH(bf16_t, 16);
    else if (Dh <= 32) GEN_LAUNCH(bf16_t, 32);
    else if (Dh <= 64) GEN_LAUNCH(bf16_t, 64);
    else GEN_LAUNCH(bf16_t, 128);
  }
#undef GEN_LAUNCH
  return check_launch("tree_attention generic");
}

// ---------------------------------------------------------------------------
// tree_attention for callers that cannot allocate: the split partials live in
// a fixed device array of the library instead of a caller workspace
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The device address of this device's copy of `scratch`, looked up once per
// device with that device current (the array's name is only a host-side
// stand-in: never pass it to a kernel or a copy).
int scratch_address(void** out) {
  int dev = -1;
  MEDUSA_HIP(hipGetDevice(&dev));
  MEDUSA_REQUIRE(dev >= 0 && dev < kMaxDevices, MEDUSA_ERR_UNSUPPORTED, "tree_attention_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    MEDUSA_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    MEDUSA_REQUIRE(p != nullptr, MEDUSA_ERR_HIP, "tree_attention_noalloc: no address for the scratch array");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MEDUSA_OK;
}

}  // namespace

extern "C" size_t tree_attention_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

extern "C" int tree_attention_noalloc(int dtype, int B, int T, int Hq, int Hkv, int Dh, const void* q, const void* Kc,
                                      const void* Vc, int64_t Lmax, int64_t L_hint, const int32_t* seq_len,
                                      const void* Kt, const void* Vt, const uint64_t* anc, float scale, void* out,
                                      hipStream_t stream) {
  const size_t need = tree_attention_workspace_size(dtype, B, T, Hq, Hkv, Dh, L_hint);
  MEDUSA_REQUIRE(need <= kNoAllocScratchBytes, MEDUSA_ERR_WORKSPACE,
                 "tree_attention_noalloc: this shape needs %zu bytes of split partials, more than the %zu-byte "
                 "static scratch; use tree_attention with a workspace",
                 need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_address(&ws);
    if (rc) return rc;
  }
  return tree_attention(dtype, B, T, Hq, Hkv, Dh, q, Kc, Vc, Lmax, L_hint, seq_len, Kt, Vt, anc, scale, out, ws,
                        need, stream);
}
