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
//  * attn_mfma -- bf16, head size 64 or 128, the streaming kernel.  One
//    workgroup (4 waves) per (sequence, KV head, row chunk of <= 256 query rows,
//    KV split).  All T*G query rows that share a KV head (G = Hq/Hkv) are served
//    by one pass over that head's keys: 64-key K and V tiles are staged in LDS
//    (double-buffered, V transposed on the way in), S^T = K Q^T and O^T += V^T P^T
//    run on 32x32x16 bf16 MFMA with fp32 accumulation, the softmax is online
//    in the log2 domain, and the tree tile is processed last with the bitset
//    mask.  KV splits write fp32 partials that attn_combine merges.
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

// --------------------------------------------------------------------------
// MFMA streaming kernel
// --------------------------------------------------------------------------
constexpr int KT = 64;        // keys per tile
constexpr int ROWS_WG = 256;  // query rows per workgroup
constexpr int NTHR = 256;

union Frag8 {
  uint4 u;
  bf16x8 v;
};

__device__ __forceinline__ bf16x8 pack8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)p[e];
  return r;
}

template <int DH>
struct AttnSmem {
  static constexpr int KP = DH + 8;  // K row pitch (elements)
  static constexpr int VP = KT + 4;  // V^T row pitch (elements)
  bf16_t k[2][KT * KP];
  bf16_t v[2][DH * VP];
};

template <int DH>
__global__ __launch_bounds__(NTHR, 1) void attn_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc, int64_t Lmax,
    const int32_t* __restrict__ seq_len, const bf16_t* __restrict__ Kt, const bf16_t* __restrict__ Vt,
    const uint64_t* __restrict__ anc, int Tn, int Hq, int Hkv, int n_rchunks, float scale_log2, int n_splits,
    bf16_t* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  using S = AttnSmem<DH>;
  constexpr int KP = S::KP, VP = S::VP;
  constexpr int NKK = DH / 16;  // k-steps of the S^T product
  constexpr int NDB = DH / 32;  // 32-row blocks of O^T
  constexpr int CPR = DH / 8;   // 16-byte chunks per K/V row
  constexpr int KPT = CPR / 4;  // keys per thread in the V transpose (4 for DH 128, 2 for DH 64)
  constexpr int KCH = KT * CPR / NTHR;  // K chunks per thread
  __shared__ S sm;

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z / n_rchunks;
  const int rchunk = blockIdx.z % n_rchunks;
  const int G = Hq / Hkv;
  const int R = Tn * G;
  const int r0 = rchunk * ROWS_WG;
  const int nr = min(ROWS_WG, R - r0);
  const int nrb = (nr + 31) >> 5;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;  // query column within a row block / key row within a key block
  const int hh = lane >> 5;  // lane half

  int64_t L = seq_len[b];
  if (L > Lmax) L = Lmax;
  if (L < 0) L = 0;
  const int tiles = (int)((L + KT - 1) / KT);
  const int tps = (tiles + n_splits - 1) / n_splits;
  const int t_begin = min(split * tps, tiles);
  const int t_end = min(t_begin + tps, tiles);
  const bool has_tree = split == n_splits - 1;
  const int ntile = (t_end - t_begin) + (has_tree ? 1 : 0);

  const size_t slab = (size_t)b * Hkv + kvh;
  const bf16_t* kc = Kc + slab * Lmax * DH;
  const bf16_t* vc = Vc + slab * Lmax * DH;
  const bf16_t* kt = Kt + slab * Tn * DH;
  const bf16_t* vt = Vt + slab * Tn * DH;

  // ---- this wave's row blocks and query fragments
  const int rbs[2] = {w, w + 4};
  bool act[2];
  int qrow[2];
  uint64_t qmask[2];
  bf16x8 qf[2][NKK];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    act[r] = rbs[r] < nrb;
    qrow[r] = r0 + rbs[r] * 32 + lq;
    const bool real = act[r] && (qrow[r] < R);
    const int node = real ? qrow[r] / G : 0;
    const int g = real ? qrow[r] % G : 0;
    qmask[r] = real ? (anc[node] & (Tn >= 64 ? ~0ull : ((1ull << Tn) - 1ull))) : 1ull;
    const bf16_t* qp = q + (((size_t)b * Tn + node) * Hq + (size_t)kvh * G + g) * DH;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      Frag8 f;
      f.u = real ? *(const uint4*)(qp + kk * 16 + hh * 8) : make_uint4(0, 0, 0, 0);
      qf[r][kk] = f.v;
    }
  }

  f32x16 o[2][NDB];
  float mrun[2], lrun[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    mrun[r] = -INFINITY;
    lrun[r] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[r][db][e] = 0.f;
  }

  // ---- tile staging: global -> registers -> LDS
  uint4 kreg[KCH];
  uint4 vreg[KPT];
  const int vkg = tid / CPR;  // V: key group (KPT keys)
  const int vch = tid % CPR;  // V: 8-dim chunk

  auto load_tile = [&](int it) {
    const bool tree = it >= (t_end - t_begin);
    const int64_t base = tree ? 0 : (int64_t)(t_begin + it) * KT;
    const int nvalid = tree ? Tn : (int)min<int64_t>(KT, L - base);
    const bf16_t* ksrc = tree ? kt : kc + base * DH;
    const bf16_t* vsrc = tree ? vt : vc + base * DH;
#pragma unroll
    for (int e = 0; e < KCH; ++e) {
      const int c = tid + e * NTHR;
      const int row = c / CPR, ch = c % CPR;
      kreg[e] = row < nvalid ? *(const uint4*)(ksrc + (size_t)row * DH + ch * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int row = vkg * KPT + e;
      vreg[e] = row < nvalid ? *(const uint4*)(vsrc + (size_t)row * DH + vch * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int e = 0; e < KCH; ++e) {
      const int c = tid + e * NTHR;
      const int row = c / CPR, ch = c % CPR;
      *(uint4*)(&sm.k[buf][row * KP + ch * 8]) = kreg[e];
    }
    // transpose: dim (vch*8 + d) gets KPT consecutive keys
    const uint32_t* vw = (const uint32_t*)vreg;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      uint16_t vals[KPT];
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        const uint32_t word = vw[e * 4 + (d >> 1)];
        vals[e] = (d & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xffff);
      }
      bf16_t* dst = &sm.v[buf][(vch * 8 + d) * VP + vkg * KPT];
      if constexpr (KPT == 4) {
        uint2 pk;
        pk.x = (uint32_t)vals[0] | ((uint32_t)vals[1] << 16);
        pk.y = (uint32_t)vals[2] | ((uint32_t)vals[3] << 16);
        *(uint2*)dst = pk;
      } else {
        *(uint32_t*)dst = (uint32_t)vals[0] | ((uint32_t)vals[1] << 16);
      }
    }
  };

  if (ntile > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < ntile; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntile) load_tile(it + 1);
    const bool tree = it >= (t_end - t_begin);
    const int64_t base = tree ? 0 : (int64_t)(t_begin + it) * KT;
    const int nvalid = tree ? Tn : (int)min<int64_t>(KT, L - base);
    const bf16_t* ks = sm.k[buf];
    const bf16_t* vs = sm.v[buf];
#pragma unroll
    for (int kb = 0; kb < KT / 32; ++kb) {
      f32x16 s[2];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[r][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        Frag8 kf;
        kf.u = *(const uint4*)(ks + (kb * 32 + lq) * KP + kk * 16 + hh * 8);
#pragma unroll
        for (int r = 0; r < 2; ++r)
          if (act[r]) s[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v, qf[r][kk], s[r], 0, 0, 0);
      }
      bf16x8 pb[2][2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (!act[r]) continue;
        float p[16];
        float mloc = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          const bool ok = tree ? ((qmask[r] >> key) & 1ull) != 0 : key < nvalid;
          p[e] = ok ? s[r][e] * scale_log2 : -INFINITY;
          mloc = fmaxf(mloc, p[e]);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const float mnew = fmaxf(mrun[r], mloc);
        const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mrun[r] - mnew);
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p[e] = (mnew == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(p[e] - mnew);
          ps += p[e];
        }
        lrun[r] = lrun[r] * alpha + ps;
        mrun[r] = mnew;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[r][db][e] *= alpha;
        pb[r][0] = pack8(p);
        pb[r][1] = pack8(p + 8);
      }
#pragma unroll
      for (int ksub = 0; ksub < 2; ++ksub) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16_t* vrow = vs + (db * 32 + lq) * VP + kb * 32 + ksub * 16 + 4 * hh;
          union {
            uint2 u[2];
            bf16x8 v;
          } vf;
          vf.u[0] = *(const uint2*)(vrow);
          vf.u[1] = *(const uint2*)(vrow + 8);
#pragma unroll
          for (int r = 0; r < 2; ++r)
            if (act[r]) o[r][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.v, pb[r][ksub], o[r][db], 0, 0, 0);
        }
      }
    }
    if (it + 1 < ntile) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (!act[r]) continue;
    const float ltot = lrun[r] + __shfl_xor(lrun[r], 32, 64);
    const bool real = qrow[r] < R;
    if (n_splits == 1) {
      if (!real) continue;
      const int node = qrow[r] / G, g = qrow[r] % G;
      bf16_t* op = out + (((size_t)b * Tn + node) * Hq + (size_t)kvh * G + g) * DH;
      const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16(o[r][db][4 * j + 0] * inv) | ((uint32_t)f32_to_bf16(o[r][db][4 * j + 1] * inv) << 16);
          pk.y = (uint32_t)f32_to_bf16(o[r][db][4 * j + 2] * inv) | ((uint32_t)f32_to_bf16(o[r][db][4 * j + 3] * inv) << 16);
          *(uint2*)(op + db * 32 + 8 * j + 4 * hh) = pk;
        }
    } else {
      if (!real) continue;
      const size_t prow = (slab * n_splits + split) * (size_t)R + qrow[r];
      float* po = ws_o + prow * DH;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float4 v4 = make_float4(o[r][db][4 * j + 0], o[r][db][4 * j + 1], o[r][db][4 * j + 2], o[r][db][4 * j + 3]);
          *(float4*)(po + db * 32 + 8 * j + 4 * hh) = v4;
        }
      if (hh == 0) {
        ws_ml[prow * 2 + 0] = mrun[r];
        ws_ml[prow * 2 + 1] = ltot;
      }
    }
  }
}

// grid (R, Hkv, B), block DH threads: merge the split partials of one query row.
template <typename T>
__global__ void attn_combine_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml, int Tn, int Hq,
                                    int Hkv, int Dh, int n_splits, T* __restrict__ out) {
  const int r = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int R = Tn * G;
  const size_t slab = (size_t)b * Hkv + kvh;
  float mt = -INFINITY;
  for (int s = 0; s < n_splits; ++s) mt = fmaxf(mt, ws_ml[((slab * n_splits + s) * R + r) * 2]);
  float lt = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const size_t pr = (slab * n_splits + s) * R + r;
    const float ms = ws_ml[pr * 2];
    if (ms != -INFINITY) lt += ws_ml[pr * 2 + 1] * __builtin_amdgcn_exp2f(ms - mt);
  }
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const int node = r / G, g = r % G;
  const size_t ooff = (((size_t)b * Tn + node) * Hq + (size_t)kvh * G + g) * Dh;
  for (int d = threadIdx.x; d < Dh; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < n_splits; ++s) {
      const size_t pr = (slab * n_splits + s) * R + r;
      const float ms = ws_ml[pr * 2];
      if (ms != -INFINITY) acc += ws_o[pr * Dh + d] * __builtin_amdgcn_exp2f(ms - mt);
    }
    Elem<T>::store(out, ooff + d, acc * inv);
  }
}

struct MfmaPlan {
  int n_rchunks, n_splits;
  size_t ws_o_bytes, ws_ml_bytes;
};

MfmaPlan mfma_plan(int B, int T, int Hq, int Hkv, int Dh, int64_t L_hint) {
  MfmaPlan p;
  const int R = T * (Hq / Hkv);
  p.n_rchunks = (R + ROWS_WG - 1) / ROWS_WG;
  const int64_t tiles = (L_hint + KT - 1) / KT;
  const int64_t units = (int64_t)B * Hkv * p.n_rchunks;
  // aim at one workgroup per CU (256 CUs), each split at least 4 tiles
  int64_t s = (256 + units - 1) / units;
  const int64_t smax = (tiles + 3) / 4;
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
    if (Dh == 128)
      hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, dim3(NTHR), 0, stream, (const bf16_t*)q, (const bf16_t*)Kc,
                         (const bf16_t*)Vc, Lmax, seq_len, (const bf16_t*)Kt, (const bf16_t*)Vt, anc, T, Hq, Hkv,
                         p.n_rchunks, sl2, p.n_splits, (bf16_t*)out, ws_o, ws_ml);
    else
      hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, dim3(NTHR), 0, stream, (const bf16_t*)q, (const bf16_t*)Kc,
                         (const bf16_t*)Vc, Lmax, seq_len, (const bf16_t*)Kt, (const bf16_t*)Vt, anc, T, Hq, Hkv,
                         p.n_rchunks, sl2, p.n_splits, (bf16_t*)out, ws_o, ws_ml);
    int rc = check_launch("tree_attention mfma");
    if (rc) return rc;
    if (p.n_splits > 1) {
      hipLaunchKernelGGL(attn_combine_kernel<bf16_t>, dim3(T * (Hq / Hkv), Hkv, B), dim3(Dh), 0, stream, ws_o, ws_ml,
                         T, Hq, Hkv, Dh, p.n_splits, (bf16_t*)out);
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
