// bf16 streaming tree attention (head size 64 or 128) on CDNA4 matrix cores.
//
// Computes, for every tree node i and query head h, softmax over the KV prefix
// plus the tree ancestors of i (page "大模型推理 memory bandwidth bound (5) -
// Medusa", section 一.2: a node only sees its predecessors; section 二.3: the
// prefix stays visible) times V.
//
// One workgroup of NW <= 8 waves per (sequence, KV head, chunk of <= 32*NW
// query rows, KV split).  The T*G query rows sharing a KV head (G = Hq/Hkv) are all served
// by a single pass over that head's keys, so K/V bytes are read from HBM once
// per KV head no matter how many query heads share them.  Wave w owns the
// 32-row block w:
//   * 64-key K and V tiles go global -> registers -> LDS, double-buffered in
//     LDS with a second tile in flight in registers (two tiles of compute hide
//     each load); V is transposed on the way in so the P.V operand reads are
//     contiguous;
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 (fp32
//     accumulation), Q fragments held in registers for the whole pass;
//   * online softmax in the log2 domain per 32-key block; O and the row sum
//     are rescaled only when the running maximum grows by more than 2^8, which
//     keeps the exponentials bounded and makes rescales rare;
//   * masks are selects: the last, ragged prefix tile by key index, the tree
//     tile (processed last) by the node's 64-bit ancestor word.
// With several KV splits each workgroup writes fp32 partials (O, m, l) that
// attn_combine merges.
#include <stdlib.h>

#include <type_traits>

#include "attn_stream.h"

namespace medusa {
namespace {

constexpr int KT = ATTN_KT;

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

__device__ __forceinline__ uint4 sel0(bool ok, uint4 v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

template <int DH>
struct StreamSmem {
  static constexpr int KP = DH + 8;  // K row pitch (elements): rows land on different banks
  static constexpr int VP = KT + 4;  // V^T row pitch (elements)
  bf16_t k[2][KT * KP];
  bf16_t v[2][DH * VP];
};

// DH head size; NW waves per workgroup (32 query rows each); PF tiles held in
// registers ahead of the LDS tile being computed (1 or 2).
template <int DH, int NW, int PF>
__global__ __launch_bounds__(NW * 64) void attn_stream_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc, int64_t Lmax,
    const int32_t* __restrict__ seq_len, const bf16_t* __restrict__ Kt, const bf16_t* __restrict__ Vt,
    const uint64_t* __restrict__ anc, int Tn, int Hq, int Hkv, int n_rchunks, float scale_log2, int n_splits,
    bf16_t* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  using S = StreamSmem<DH>;
  constexpr int NTHR = NW * 64;
  constexpr int ROWS_WG = NW * 32;
  constexpr int KP = S::KP, VP = S::VP;
  constexpr int NKK = DH / 16;           // k-steps of the S^T product
  constexpr int NDB = DH / 32;           // 32-row blocks of O^T
  constexpr int CPR = DH / 8;            // 16-byte chunks per K/V row
  constexpr int KCH = KT * CPR / NTHR;   // K chunks per thread
  constexpr int KPT = KT * CPR / NTHR;   // keys per thread in the V transpose (1, 2 or 4)
  constexpr float RESCALE_SLACK = 8.0f;  // log2 units
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
  const int lq = lane & 31;  // query column of the row block / key row of a key block
  const int hh = lane >> 5;  // lane half

  int64_t L = seq_len[b];
  if (L > Lmax) L = Lmax;
  if (L < 0) L = 0;
  const int tiles = (int)((L + KT - 1) / KT);
  const int tps = (tiles + n_splits - 1) / n_splits;
  const int t_begin = min(split * tps, tiles);
  const int t_end = min(t_begin + tps, tiles);
  const int npre = t_end - t_begin;
  const bool has_tree = split == n_splits - 1;
  const int ntile = npre + (has_tree ? 1 : 0);

  const size_t slab = (size_t)b * Hkv + kvh;
  const bf16_t* kc = Kc + slab * Lmax * DH;
  const bf16_t* vc = Vc + slab * Lmax * DH;
  const bf16_t* kt = Kt + slab * Tn * DH;
  const bf16_t* vt = Vt + slab * Tn * DH;
  const uint64_t tmask = Tn >= 64 ? ~0ull : ((1ull << Tn) - 1ull);

  // ---- this wave's row block: query fragments (B operand of S^T), mask word
  const bool act = __builtin_amdgcn_readfirstlane((int)(w < nrb)) != 0;  // wave-uniform
  const int qrow = r0 + w * 32 + lq;
  const bool real = act && qrow < R;
  const int qnode = real ? qrow / G : 0;
  const int qg = real ? qrow % G : 0;
  const uint64_t qmask = real ? (anc[qnode] & tmask) : 1ull;
  bf16x8 qf[NKK];
  {
    const bf16_t* qp = q + (((size_t)b * Tn + qnode) * Hq + (size_t)kvh * G + qg) * DH;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      Frag8 f;
      f.u = sel0(real, *(const uint4*)(qp + kk * 16 + hh * 8));
      qf[kk] = f.v;
    }
  }
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  // ---- tile staging
  struct Stage {
    uint4 k[KCH];
    uint4 v[KPT];
  };
  Stage R0;
  [[maybe_unused]] Stage R1;
  const int vkg = tid / CPR;  // V: group of KPT consecutive keys
  const int vch = tid % CPR;  // V: 8-dim chunk

  auto load_tile = [&](int it, Stage& st) {
    const bool tree = it >= npre;
    const int64_t base = tree ? 0 : (int64_t)(t_begin + it) * KT;
    const int nvalid = tree ? Tn : (int)min<int64_t>(KT, L - base);
    const bf16_t* ksrc = tree ? kt : kc + base * DH;
    const bf16_t* vsrc = tree ? vt : vc + base * DH;
    // rows past nvalid read row 0 (in bounds) and are zeroed by a select
#pragma unroll
    for (int e = 0; e < KCH; ++e) {
      const int c = tid + e * NTHR;
      const int row = c / CPR, ch = c % CPR;
      const bool ok = row < nvalid;
      st.k[e] = sel0(ok, *(const uint4*)(ksrc + (size_t)(ok ? row : 0) * DH + ch * 8));
    }
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int row = vkg * KPT + e;
      const bool ok = row < nvalid;
      st.v[e] = sel0(ok, *(const uint4*)(vsrc + (size_t)(ok ? row : 0) * DH + vch * 8));
    }
  };
  auto store_tile = [&](const Stage& st, int buf) {
#pragma unroll
    for (int e = 0; e < KCH; ++e) {
      const int c = tid + e * NTHR;
      const int row = c / CPR, ch = c % CPR;
      *(uint4*)(&sm.k[buf][row * KP + ch * 8]) = st.k[e];
    }
    // transpose: V^T row (vch*8 + d) gets this thread's KPT consecutive keys
    const uint32_t* vw = (const uint32_t*)st.v;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      uint32_t h[KPT];
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        const uint32_t word = vw[e * 4 + (d >> 1)];
        h[e] = (d & 1) ? (word >> 16) : (word & 0xffffu);
      }
      bf16_t* dst = &sm.v[buf][(vch * 8 + d) * VP + vkg * KPT];
      if constexpr (KPT == 8) {
        // V^T rows are 8-byte aligned (pitch 68 elements)
        *(uint2*)dst = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        *(uint2*)(dst + 4) = make_uint2(h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      } else if constexpr (KPT == 4) {
        *(uint2*)dst = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      } else if constexpr (KPT == 2) {
        *(uint32_t*)dst = h[0] | (h[1] << 16);
      } else {
        *dst = (bf16_t)h[0];
      }
    }
  };

  auto compute_tile = [&](int it, int buf) {
    if (!act) return;
    const bool tree = it >= npre;
    const int64_t base = tree ? 0 : (int64_t)(t_begin + it) * KT;
    const int nvalid = tree ? Tn : (int)min<int64_t>(KT, L - base);
    const bool need_mask = tree || nvalid < KT;
    const bf16_t* ks = sm.k[buf];
    const bf16_t* vs = sm.v[buf];
#pragma unroll
    for (int kb = 0; kb < KT / 32; ++kb) {
      // all LDS fragment reads of the block are issued up front: the K reads
      // overlap each other, the V reads overlap the S product and the softmax
      Frag8 kf[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) kf[kk].u = *(const uint4*)(ks + (kb * 32 + lq) * KP + kk * 16 + hh * 8);
      union VF {
        uint2 u[2];
        bf16x8 v;
      } vf[2][NDB];
#pragma unroll
      for (int ksub = 0; ksub < 2; ++ksub)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16_t* vrow = vs + (db * 32 + lq) * VP + kb * 32 + ksub * 16 + 4 * hh;
          vf[ksub][db].u[0] = *(const uint2*)(vrow);
          vf[ksub][db].u[1] = *(const uint2*)(vrow + 8);
        }
      // S^T (32 keys x 32 queries) = K Q^T.  With few waves per SIMD, two
      // interleaved accumulation chains (even / odd k-steps) keep consecutive
      // MFMAs independent; the 8-wave kernel has other waves to overlap and no
      // registers to spare.
      f32x16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
      if constexpr (NW <= 4) {
        f32x16 s1;
#pragma unroll
        for (int e = 0; e < 16; ++e) s1[e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; kk += 2) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk].v, qf[kk], s, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk + 1].v, qf[kk + 1], s1, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] += s1[e];
      } else {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk].v, qf[kk], s, 0, 0, 0);
      }
      // lane holds keys kb*32 + 8j + 4*hh + i (value s[4j+i]) of query lq
      if (need_mask) {
        // one 32-bit validity word for the block's keys, then a bit test per key
        const int nv = nvalid - kb * 32;
        const uint32_t kbits = tree ? (uint32_t)(qmask >> (kb * 32))
                                    : (nv >= 32 ? 0xffffffffu : (nv <= 0 ? 0u : ((1u << nv) - 1u)));
        const uint32_t mine = kbits >> (4 * hh);
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = ((mine >> (8 * (e >> 2) + (e & 3))) & 1u) ? s[e] : -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mt = mx * scale_log2;
      if (mt > mrun + RESCALE_SLACK) {
        const float alpha = __builtin_amdgcn_exp2f(mrun - mt);
        lrun *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
        mrun = mt;
      }
      const float negm = mrun == -INFINITY ? 0.f : -mrun;
      float p[16];
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(s[e], scale_log2, negm));
        ps += p[e];
      }
      lrun += ps;
      // P^T B operand: k-slot t of lane half hh <-> key 16*ksub + 8*(t/4) + 4*hh + t%4
      const bf16x8 pb0 = pack8(p), pb1 = pack8(p + 8);
#pragma unroll
      for (int ksub = 0; ksub < 2; ++ksub)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ksub][db].v, ksub ? pb1 : pb0, o[db], 0, 0, 0);
    }
  };

  if constexpr (PF == 2) {
    // tile it in LDS buffer (it & 1), tile it+1 in registers, tile it+2 being
    // fetched; unrolled by two so the register stages are static
    if (ntile > 0) {
      load_tile(0, R0);
      store_tile(R0, 0);
    }
    if (ntile > 1) load_tile(1, R1);
    __syncthreads();
    int it = 0;
    for (; it + 1 < ntile; it += 2) {
      if (it + 2 < ntile) load_tile(it + 2, R0);
      compute_tile(it, 0);
      store_tile(R1, 1);
      __syncthreads();
      if (it + 3 < ntile) load_tile(it + 3, R1);
      compute_tile(it + 1, 1);
      if (it + 2 < ntile) store_tile(R0, 0);
      __syncthreads();
    }
    if (it < ntile) compute_tile(it, 0);
  } else {
    // tile it in LDS buffer (it & 1) while tile it+1 is fetched into registers
    if (ntile > 0) {
      load_tile(0, R0);
      store_tile(R0, 0);
    }
    __syncthreads();
    for (int it = 0; it < ntile; ++it) {
      if (it + 1 < ntile) load_tile(it + 1, R0);
      compute_tile(it, it & 1);
      if (it + 1 < ntile) store_tile(R0, (it + 1) & 1);
      __syncthreads();
    }
  }

  // ---- epilogue: O^T lane layout is rows dh = db*32 + 8j + 4*hh + i of query lq
  if (!real) return;
  const float ltot = lrun + __shfl_xor(lrun, 32, 64);
  if (n_splits == 1) {
    bf16_t* op = out + (((size_t)b * Tn + qnode) * Hq + (size_t)kvh * G + qg) * DH;
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(o[db][4 * j + 0] * inv) | ((uint32_t)f32_to_bf16(o[db][4 * j + 1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16(o[db][4 * j + 2] * inv) | ((uint32_t)f32_to_bf16(o[db][4 * j + 3] * inv) << 16);
        *(uint2*)(op + db * 32 + 8 * j + 4 * hh) = pk;
      }
  } else {
    const size_t prow = (slab * n_splits + split) * (size_t)R + qrow;
    float* po = ws_o + prow * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(float4*)(po + db * 32 + 8 * j + 4 * hh) =
            make_float4(o[db][4 * j + 0], o[db][4 * j + 1], o[db][4 * j + 2], o[db][4 * j + 3]);
    if (hh == 0) {
      ws_ml[prow * 2 + 0] = mrun;
      ws_ml[prow * 2 + 1] = ltot;
    }
  }
}

}  // namespace

// Waves per workgroup: one per 32-row block of the rows sharing a KV head, at
// least 2 and at most 8 (R <= 64 -> 2, R <= 128 -> 4, else 8), always with two
// register tiles in flight.  MEDUSA_ATTN_WAVES = 2 | 4 | 8 forces a width for
// tuning runs.
int attn_stream_waves(int R) {
  static const int forced = [] {
    const char* e = getenv("MEDUSA_ATTN_WAVES");
    const int v = e ? atoi(e) : 0;
    return v == 2 || v == 4 || v == 8 ? v : 0;
  }();
  if (forced) return forced;
  return R <= 64 ? 2 : (R <= 128 ? 4 : 8);
}

template <int NW, int PF>
static void launch_v(int Dh, dim3 grid, hipStream_t stream, const bf16_t* q, const bf16_t* Kc, const bf16_t* Vc,
                     int64_t Lmax, const int32_t* seq_len, const bf16_t* Kt, const bf16_t* Vt, const uint64_t* anc,
                     int T, int Hq, int Hkv, int n_rchunks, float scale_log2, int n_splits, bf16_t* out, float* ws_o,
                     float* ws_ml) {
  if (Dh == 128)
    hipLaunchKernelGGL((attn_stream_kernel<128, NW, PF>), grid, dim3(NW * 64), 0, stream, q, Kc, Vc, Lmax, seq_len,
                       Kt, Vt, anc, T, Hq, Hkv, n_rchunks, scale_log2, n_splits, out, ws_o, ws_ml);
  else
    hipLaunchKernelGGL((attn_stream_kernel<64, NW, PF>), grid, dim3(NW * 64), 0, stream, q, Kc, Vc, Lmax, seq_len,
                       Kt, Vt, anc, T, Hq, Hkv, n_rchunks, scale_log2, n_splits, out, ws_o, ws_ml);
}

int launch_attn_stream(int Dh, int nw, dim3 grid, hipStream_t stream, const bf16_t* q, const bf16_t* Kc,
                       const bf16_t* Vc, int64_t Lmax, const int32_t* seq_len, const bf16_t* Kt, const bf16_t* Vt,
                       const uint64_t* anc, int T, int Hq, int Hkv, int n_rchunks, float scale_log2, int n_splits,
                       bf16_t* out, float* ws_o, float* ws_ml) {
  if (Dh != 128 && Dh != 64) return fail(MEDUSA_ERR_UNSUPPORTED, "tree_attention: streaming kernel takes Dh 64 or 128");
  if (nw == 2)
    launch_v<2, 2>(Dh, grid, stream, q, Kc, Vc, Lmax, seq_len, Kt, Vt, anc, T, Hq, Hkv, n_rchunks, scale_log2,
                   n_splits, out, ws_o, ws_ml);
  else if (nw == 4)
    launch_v<4, 2>(Dh, grid, stream, q, Kc, Vc, Lmax, seq_len, Kt, Vt, anc, T, Hq, Hkv, n_rchunks, scale_log2,
                   n_splits, out, ws_o, ws_ml);
  else
    launch_v<8, 2>(Dh, grid, stream, q, Kc, Vc, Lmax, seq_len, Kt, Vt, anc, T, Hq, Hkv, n_rchunks, scale_log2,
                   n_splits, out, ws_o, ws_ml);
  return check_launch("tree_attention stream");
}

}  // namespace medusa
