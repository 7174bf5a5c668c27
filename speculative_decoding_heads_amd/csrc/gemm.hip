// Dense products C = A W^T with fused epilogues, for the Medusa heads and the
// verify forward.
//
// The Medusa head of the page "大模型推理 memory bandwidth bound (5) - Medusa"
// (section 一.1) is z = SiLU(W1 h) + h followed by W2 z; the verify forward
// (section 二.5) runs the base model's projections on all T tree tokens at once.
// Both are weight-streaming products with few rows (M = batch or batch*T), so
// the bf16 kernel is built for HBM streaming, not for square tiles:
//
//  * bf16, every M (one 64-row activation tile per workgroup, rows past M
//    re-reading row M - 1): gemm_dma_kernel when K % 64 == 0 (both operands
//    into an LDS ring by direct loads), gemm_lds_kernel otherwise (weights
//    through registers, activation in LDS); both below.
//  * bf16 register kernel (gemm_bf16_kernel; taken only under the tuning
//    variables for M <= 32): a wave owns 32 or 64 rows of W and up to 64 rows of A; W is
//    the MFMA A-operand (16x16x32 bf16, fp32 accumulate) so each lane loads 16
//    contiguous bytes of one W row per k-step.  The four waves of a workgroup
//    take neighbouring W rows over the same k range (their A loads coincide and
//    hit in L1), each with a two-stage register pipeline.  When the grid would
//    be too small to keep ~8 waves per CU busy the K range is also split across
//    workgroups; a second kernel then adds the fp32 partials in a fixed order
//    and applies the epilogue.
//  * fp32: one thread per output with a sequential k loop, so a row's result
//    does not depend on M or on the row's position (plain decode and tree
//    verification agree bit for bit).
//
// Epilogues: store fp32; store in dtype; residual add; Medusa residual
// (A[m, n mod K] + SiLU(acc), the head's h + SiLU(W1 h) with W1 of size K x K);
// SwiGLU on row-interleaved gate/up weights (row 2j = gate j, row 2j+1 = up j).
#include <stdlib.h>

#include <type_traits>
#include <utility>

#include "common.h"
#include "medusa_model.h"

using namespace medusa;

namespace {

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

struct EpiArgs {
  int mode;
  void* C;
  int64_t ldc;
  const void* R;
  int64_t ldr;
  const void* A;  // for MEDUSA_EPI_SILU_RESID_A
  int64_t lda;
  int K;
  int part_only;  // bf16 kernels: always leave fp32 partials (a fused consumer reduces them)
  // EPI_QKV_ROPE (gemm_lds_kernel with NR == 1, SK == 1): rotary embedding and
  // the q / K / V split of a fused [(Hq + 2 Hkv) * Dh, d] projection
  const int32_t* pos;
  const float* cos_t;
  const float* sin_t;
  int max_pos, T, Hq, Hkv, Dh;
  bf16_t *q_out, *k_out, *v_out;
};

// Internal epilogue mode (not in the public enum): see EpiArgs.
constexpr int EPI_QKV_ROPE = 100;

// Apply the epilogue to a pair-capable element set: value v at (m, n).  For
// SWIGLU the caller passes gate (n even) and up (n+1) together.
template <typename T>
__device__ __forceinline__ void epi_store(const EpiArgs& e, int m, int n, float v) {
  switch (e.mode) {
    case MEDUSA_EPI_F32:
      ((float*)e.C)[(size_t)m * e.ldc + n] = v;
      break;
    case MEDUSA_EPI_STORE:
      Elem<T>::store((T*)e.C, (size_t)m * e.ldc + n, v);
      break;
    case MEDUSA_EPI_RESID: {
      const float r = Elem<T>::load((const T*)e.R, (size_t)m * e.ldr + n);
      Elem<T>::store((T*)e.C, (size_t)m * e.ldc + n, r + v);
      break;
    }
    case MEDUSA_EPI_SILU_RESID_A: {
      const float r = Elem<T>::load((const T*)e.A, (size_t)m * e.lda + (n % e.K));
      Elem<T>::store((T*)e.C, (size_t)m * e.ldc + n, r + silu(v));
      break;
    }
    default:
      break;
  }
}

template <typename T>
__device__ __forceinline__ void epi_swiglu(const EpiArgs& e, int m, int j, float g, float u) {
  Elem<T>::store((T*)e.C, (size_t)m * e.ldc + j, silu(g) * u);
}

// ---------------------------------------------------------------------------
// fp32 (and generic) VALU kernel: one thread per output (m, n) or gate/up pair.
// grid (ceil(Nout/64), ceil(M/4), batch), block (64, 4)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void gemm_valu_kernel(int M, int N, int K, const T* __restrict__ A, int64_t lda,
                                                        int64_t sA, const T* __restrict__ W, int64_t sW,
                                                        EpiArgs e, int64_t sC, int64_t sR) {
  const int bz = blockIdx.z;
  A += bz * sA;
  W += bz * sW;
  EpiArgs eb = e;
  eb.C = (char*)e.C + bz * sC * (e.mode == MEDUSA_EPI_F32 ? 4 : (int64_t)sizeof(T));
  if (e.R) eb.R = (const char*)e.R + bz * sR * (int64_t)sizeof(T);
  eb.A = A;
  const int m = blockIdx.y * 4 + threadIdx.y;
  const int nout = blockIdx.x * 64 + threadIdx.x;
  if (m >= M) return;
  const T* a = A + (size_t)m * lda;
  if (e.mode == MEDUSA_EPI_SWIGLU) {
    if (nout >= N / 2) return;
    const T* wg = W + (size_t)(2 * nout) * K;
    const T* wu = wg + K;
    float g = 0.f, u = 0.f;
    for (int k = 0; k < K; ++k) {
      const float av = Elem<T>::load(a, k);
      g += av * Elem<T>::load(wg, k);
      u += av * Elem<T>::load(wu, k);
    }
    epi_swiglu<T>(eb, m, nout, g, u);
    return;
  }
  if (nout >= N) return;
  const T* w = W + (size_t)nout * K;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc += Elem<T>::load(a, k) * Elem<T>::load(w, k);
  epi_store<T>(eb, m, nout, acc);
}

// ---------------------------------------------------------------------------
// bf16 MFMA streaming kernel
// ---------------------------------------------------------------------------
constexpr int GK = 32;     // k per MFMA step (16x16x32 bf16)
constexpr int GTHR = 256;  // 4 waves
constexpr int GM = 64;     // A rows per tile (max)

union F8 {
  uint4 u;
  bf16x8 v;
};

// Four bf16 values (round to nearest even) as one 8-byte word, and back.
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  uint2 w;
  w.x = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  w.y = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
  return w;
}
__device__ __forceinline__ void unpack_bf16x4(uint2 w, float (&v)[4]) {
  v[0] = bf16_to_f32((bf16_t)(w.x & 0xffffu));
  v[1] = bf16_to_f32((bf16_t)(w.x >> 16));
  v[2] = bf16_to_f32((bf16_t)(w.y & 0xffffu));
  v[3] = bf16_to_f32((bf16_t)(w.y >> 16));
}

// Write a wave's (NR*16) x (MB*16) accumulator tile: fp32 partials when the
// K range is split (layout [batch][SK][M][N]), else the epilogue.  C layout of
// the 16x16 MFMA: acc[i][j][r] is W row n0 + 16i + 4*lg + r, A row m0 + 16j + l16,
// so a lane holds four consecutive outputs of one row: they are written (and a
// residual read) as one 16-, 8- or 4-byte access when the row stride and base
// alignment allow, else element by element; the values are the same either way.
template <int NR, int MB>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[NR][MB], int n0, int m0, int M, int N, int SK, int ks,
                                           int bz, const EpiArgs& e, int64_t sC, int64_t sR, const bf16_t* A,
                                           float* __restrict__ part, int l16, int lg) {
  if (SK > 1 || e.part_only) {
    float* pp = part + (((size_t)bz * SK + ks) * M) * N;
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int m = m0 + j * 16 + l16;
        if (m >= M) continue;
        const int nb = n0 + i * 16 + 4 * lg;
        float* dst = pp + (size_t)m * N + nb;
        if (vec && nb + 3 < N) {
          *(float4*)dst = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb + r < N) dst[r] = acc[i][j][r];
        }
      }
    return;
  }
  EpiArgs eb = e;
  eb.C = (char*)e.C + bz * sC * (e.mode == MEDUSA_EPI_F32 ? 4 : 2);
  if (e.R) eb.R = (const char*)e.R + bz * sR * 2;
  eb.A = A;
  const uintptr_t cbase = (uintptr_t)eb.C;
  bool vec;
  switch (e.mode) {
    case MEDUSA_EPI_F32: vec = (e.ldc & 3) == 0 && (cbase & 15) == 0; break;
    case MEDUSA_EPI_SWIGLU: vec = (e.ldc & 1) == 0 && (cbase & 3) == 0; break;
    case MEDUSA_EPI_STORE: vec = (e.ldc & 3) == 0 && (cbase & 7) == 0; break;
    case MEDUSA_EPI_RESID:
      vec = (e.ldc & 3) == 0 && (cbase & 7) == 0 && (e.ldr & 3) == 0 && ((uintptr_t)eb.R & 7) == 0;
      break;
    case MEDUSA_EPI_SILU_RESID_A:
      vec = (e.ldc & 3) == 0 && (cbase & 7) == 0 && (e.lda & 3) == 0 && ((uintptr_t)A & 7) == 0 && (e.K & 3) == 0;
      break;
    default: vec = false; break;
  }
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int m = m0 + j * 16 + l16;
      if (m >= M) continue;
      const int nb = n0 + i * 16 + 4 * lg;
      const float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if (e.mode == MEDUSA_EPI_SWIGLU) {
        if (vec && nb + 3 < N) {
          bf16_t* dst = (bf16_t*)eb.C + (size_t)m * e.ldc + nb / 2;
          *(uint32_t*)dst = (uint32_t)f32_to_bf16(silu(v[0]) * v[1]) | ((uint32_t)f32_to_bf16(silu(v[2]) * v[3]) << 16);
        } else {
          if (nb + 1 < N) epi_swiglu<bf16_t>(eb, m, nb / 2, v[0], v[1]);
          if (nb + 3 < N) epi_swiglu<bf16_t>(eb, m, nb / 2 + 1, v[2], v[3]);
        }
      } else if (vec && nb + 3 < N) {
        if (e.mode == MEDUSA_EPI_F32) {
          *(float4*)((float*)eb.C + (size_t)m * e.ldc + nb) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          float o[4] = {v[0], v[1], v[2], v[3]};
          if (e.mode == MEDUSA_EPI_RESID) {
            float r[4];
            unpack_bf16x4(*(const uint2*)((const bf16_t*)eb.R + (size_t)m * e.ldr + nb), r);
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = r[q] + o[q];
          } else if (e.mode == MEDUSA_EPI_SILU_RESID_A) {
            float r[4];
            unpack_bf16x4(*(const uint2*)(A + (size_t)m * e.lda + (nb % e.K)), r);
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = r[q] + silu(o[q]);
          }
          *(uint2*)((bf16_t*)eb.C + (size_t)m * e.ldc + nb) = pack_bf16x4(o[0], o[1], o[2], o[3]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb + r < N) epi_store<bf16_t>(eb, m, nb + r, v[r]);
      }
    }
}

// Positions of a lane's four rows (m0 + 16j + l16; rows past M read row M-1's)
// for the rotary epilogue, which clamps them.  The kernels load them before the
// product loop and use them only in the epilogue, so the loads complete under
// the loop and the table loads need no dependent round trip.
__device__ __forceinline__ void rope_positions(const EpiArgs& e, int m0, int M, int l16, int (&p)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = e.pos[min(m0 + j * 16 + l16, M - 1)];
}

// Rotary embedding + q / K / V split for a wave's 16 x 64 tile of the fused
// projection (tile mapping of EPI_QKV_ROPE in gemm_lds_kernel).  The partner
// tile (wave w ^ 1) is exchanged through LDS; every wave of the workgroup
// calls this (it holds two barriers).  Rotate-half: for i < Dh/2,
// y[i] = x[i] cos - x[i + Dh/2] sin, y[i + Dh/2] = x[i + Dh/2] cos + x[i] sin,
// at the row's position p (rope_positions), clamped to [0, max_pos); V rows
// are stored as they are.
// The cos / sin loads go out before the exchange and land during it.
__device__ __forceinline__ void rope_epilogue(const f32x4 (&acc)[1][4], char* lds, int w, int n0, int m0, int M,
                                              const EpiArgs& e, int l16, int lg, const int (&p)[4]) {
  const int Dh = e.Dh, half = Dh / 2;
  const int hd = n0 / Dh, within = n0 % Dh;
  const int hf = within >= half;                     // second half of the head
  const int i0 = (hf ? within - half : within) + 4 * lg;  // first of this lane's 4 dims (in the half)
  const bool rot = hd < e.Hq + e.Hkv;                // q or K rows (wave-uniform)
  float cs[4][4], sn[4][4];
  if (rot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pj = p[j] < 0 ? 0 : (p[j] >= e.max_pos ? e.max_pos - 1 : p[j]);
      const size_t off = (size_t)pj * half + i0;
#pragma unroll
      for (int r = 0; r < 4; ++r) cs[j][r] = e.cos_t[off + r], sn[j][r] = e.sin_t[off + r];
    }
  }
  float* xs = (float*)lds;  // [4 waves][16 rows][64 columns]
  __syncthreads();          // every wave is done with the A buffers
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) xs[(w * 16 + 4 * lg + r) * 64 + j * 16 + l16] = acc[0][j][r];
  __syncthreads();
  const int partner = w ^ 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + j * 16 + l16;
    if (m >= M) continue;
    const int b = m / e.T, t = m % e.T;
    float y[4];
    bf16_t* dst;
    if (rot) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float own = acc[0][j][r];
        const float par = xs[(partner * 16 + 4 * lg + r) * 64 + j * 16 + l16];
        // first half: own = x[i], par = x[i + half]; second half: the reverse
        y[r] = hf ? own * cs[j][r] + par * sn[j][r] : own * cs[j][r] - par * sn[j][r];
      }
      const int dim = hf * half + i0;
      dst = hd < e.Hq ? e.q_out + (((size_t)b * e.T + t) * e.Hq + hd) * Dh + dim
                      : e.k_out + (((size_t)b * e.Hkv + (hd - e.Hq)) * e.T + t) * Dh + dim;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = acc[0][j][r];
      dst = e.v_out + (((size_t)b * e.Hkv + (hd - e.Hq - e.Hkv)) * e.T + t) * Dh + within + 4 * lg;
    }
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(y[0]) | ((uint32_t)f32_to_bf16(y[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16(y[2]) | ((uint32_t)f32_to_bf16(y[3]) << 16);
    *(uint2*)dst = pk;
  }
}

// Each wave owns an (NR*16 W rows) x (MB*16 A rows) output tile.  With KW the
// four waves of a workgroup cover consecutive k ranges of the same tile and are
// summed through LDS in wave order; without it they own four neighbouring W
// tiles over the same k range (their A loads coincide and hit in L1).  Loads run
// two pipeline stages of U k-steps ahead: the next stage is issued before the
// current one is multiplied.  When the grid is split along K (SK > 1) the fp32
// partials are summed by splitk_reduce_kernel.
// grid (N tiles of (KW ? 1 : 4)*NR*16 rows, m tiles * SK, batch).
template <int MB, int NR, int U, bool KW>
__global__ __launch_bounds__(GTHR) void gemm_bf16_kernel(int M, int N, int K, const bf16_t* __restrict__ A, int64_t lda,
                                                         int64_t sA, const bf16_t* __restrict__ W, int64_t sW,
                                                         int SK, EpiArgs e, int64_t sC, int64_t sR,
                                                         float* __restrict__ part) {
  constexpr int TN = NR * 16, TM = MB * 16;
  __shared__ float red[KW ? 3 : 1][KW ? TN * TM : 1];
  const int bz = blockIdx.z;
  const int nt = blockIdx.x;
  const int mt = blockIdx.y / SK;
  const int ks = blockIdx.y % SK;
  // the wave index is uniform: keep it (and the k range below) in scalar registers
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  A += bz * sA;
  W += bz * sW;
  const int n0 = (KW ? nt : nt * 4 + w) * TN, m0 = mt * GM;
  const int nchunks = (K / GK) / U;
  const int parts = KW ? SK * 4 : SK, pi = KW ? ks * 4 + w : ks;
  const int c0 = (int)((int64_t)nchunks * pi / parts), c1 = (int)((int64_t)nchunks * (pi + 1) / parts);

  // rows past N / M are clamped to the last row; their results are discarded
  const bf16_t* wrow[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int n = min(n0 + i * 16 + l16, N - 1);
    wrow[i] = W + (size_t)n * K + lg * 8;
  }
  const bf16_t* arow[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int m = min(m0 + j * 16 + l16, M - 1);
    arow[j] = A + (size_t)m * lda + lg * 8;
  }
  f32x4 acc[NR][MB];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    F8 w[U][NR];
    F8 a[U][MB];
  };
  Stage S0, S1;
  // tiles start their k walk at different chunks (see gemm_lds_kernel)
  const int nck = c1 - c0;
  const int rot = nck > 0 ? (int)(((unsigned)nt * 37u) % (unsigned)nck) : 0;
  auto load = [&](Stage& s, int c) {
    int y = c - c0 + rot;
    if (y >= nck) y -= nck;
    const int k = (c0 + y) * U * GK;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int i = 0; i < NR; ++i) s.w[u][i].u = *(const uint4*)(wrow[i] + k + u * GK);
#pragma unroll
      for (int j = 0; j < MB; ++j) s.a[u][j].u = *(const uint4*)(arow[j] + k + u * GK);
    }
  };
  auto comp = [&](const Stage& s) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s.w[u][i].v, s.a[u][j].v, acc[i][j], 0, 0, 0);
  };
  // Loads past the wave's last chunk are clamped to that chunk (cache hits, never
  // multiplied) so the loop body has no branches around its loads.
  if (c0 < c1) {
    load(S0, c0);
    load(S1, min(c0 + 1, c1 - 1));
    int c = c0;
    // sched_barrier keeps the compiler from sinking a stage's loads below the
    // next stage's multiplies (which would serialise load latency)
    for (; c + 1 < c1; c += 2) {
      comp(S0);
      __builtin_amdgcn_sched_barrier(0);
      load(S0, min(c + 2, c1 - 1));
      __builtin_amdgcn_sched_barrier(0);
      comp(S1);
      __builtin_amdgcn_sched_barrier(0);
      load(S1, min(c + 3, c1 - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c < c1) comp(S0);
  }

  // C layout: acc[i][j][r] is W row n0 + 16i + 4*lg + r, A row m0 + 16j + l16
  if (KW) {
    if (w > 0) {
      float* dst = red[w - 1];
#pragma unroll
      for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[(i * 16 + 4 * lg + r) * TM + j * 16 + l16] = acc[i][j][r];
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] += red[q][(i * 16 + 4 * lg + r) * TM + j * 16 + l16];
  }
  store_tile<NR, MB>(acc, n0, m0, M, N, SK, ks, bz, e, sC, sR, A, part, l16, lg);
}

// 64-row activation tile kernel (K % 64 != 0).  The NWV waves of a workgroup (4, or 3 when 96-row
// workgroup tiles spread a product more evenly over the CUs) own neighbouring
// (NR*16)-row W tiles and walk the same k range; the workgroup stages the 64 A
// rows of each chunk (U k-steps) once in LDS, so A costs one global read per
// workgroup instead of one per wave (re-reading A per wave caps these products
// at about half the HBM rate).  Per chunk and wave:
//   * W fragments go straight from global memory to registers, NS chunks ahead;
//   * A goes global -> registers (NS chunks ahead) -> LDS two chunks ahead,
//     through three LDS buffers, with one barrier per chunk;
//   * the A fragments of the next chunk are read from LDS before the current
//     chunk's MFMAs are issued, so LDS latency hides behind them (with one
//     workgroup per CU there is no other wave to cover it).
// Staged rows are padded by 16 bytes so the 16 rows that one ds_read_b128
// touches fall in distinct banks.  A K split across workgroups (SK > 1) leaves
// fp32 partials.  grid (N tiles of NWV*NR*16 rows, m tiles * SK, batch).
template <int NR, int U, int NS, int NWV>
__global__ __launch_bounds__(NWV * 64) void gemm_lds_kernel(int M, int N, int K, const bf16_t* __restrict__ A,
                                                            int64_t lda, int64_t sA, const bf16_t* __restrict__ W,
                                                            int64_t sW, int SK, EpiArgs e, int64_t sC, int64_t sR,
                                                            float* __restrict__ part) {
  constexpr int MB = 4, TN = NR * 16;
  constexpr int NTHR = NWV * 64;
  constexpr int ROWB = U * GK * 2 + 16;  // bytes per staged A row
  constexpr int PPR = U * GK * 2 / 16;   // 16-byte pieces per A row and chunk
  constexpr int NPC = GM * PPR;          // pieces per chunk
  constexpr int PPT = (NPC + NTHR - 1) / NTHR;  // pieces per thread and chunk (the last ones partly idle)
  constexpr int BUFB = GM * ROWB;
  static_assert(NS >= 4 && NS % 2 == 0, "the staging distance needs NS >= 4, even");
  // three A buffers; the rotary epilogue reuses them for a 4 x 16 x 64 fp32 exchange
  __shared__ __align__(16) char lds[3 * BUFB > 16384 ? 3 * BUFB : 16384];
  const int bz = blockIdx.z;
  const int nt = blockIdx.x;
  const int mt = blockIdx.y / SK;
  const int ks = blockIdx.y % SK;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  A += bz * sA;
  W += bz * sW;
  // EPI_QKV_ROPE maps the four 16-row wave tiles to two blocks of the first
  // half of one head's rows and the same blocks of the second half (waves
  // w and w ^ 1 hold the two rotary partners of the same dimensions)
  // With three waves (equal numbers of rotary pairs and V blocks, as in
  // multi-head attention) waves 0 and 1 hold one pair of q or k blocks and
  // wave 2 one 16-row block of V, so every workgroup has 48 rows.
  const bool rope = NR == 1 && (NWV == 4 || NWV == 3) && e.mode == EPI_QKV_ROPE;
  int n0 = (nt * NWV + w) * TN;
  if (rope) {
    if constexpr (NWV == 3) {
      const int pairs_per_head = e.Dh / 32;
      n0 = w < 2 ? (nt / pairs_per_head) * e.Dh + w * (e.Dh / 2) + (nt % pairs_per_head) * 16
                 : (e.Hq + e.Hkv) * e.Dh + nt * 16;
    } else {
      const int wg_per_head = e.Dh / 64, hd = nt / wg_per_head, sub = nt % wg_per_head;
      n0 = hd * e.Dh + (w & 1) * (e.Dh / 2) + (sub * 2 + (w >> 1)) * 16;
    }
  }
  const int m0 = mt * GM;
  // rotary rows' positions, loaded ahead of the product loop
  int rpos[4] = {0, 0, 0, 0};
  if (rope) rope_positions(e, m0, M, l16, rpos);
  const int nchunks = (K / GK) / U;
  const int c0 = (int)((int64_t)nchunks * ks / SK), c1 = (int)((int64_t)nchunks * (ks + 1) / SK);
  const int per = c1 - c0;  // chunks of this workgroup (uniform)
  // Workgroups start their k walk at different chunks (rotated by the W tile
  // index): walking in step, all of them would hit the same column offset of
  // their W rows at once and crowd the same memory channels.  Workgroups of one
  // W tile (several m tiles) keep the same order so they share its lines in
  // L2.  The rotation only changes the order of the k sum, fixed for a shape.
  const int rot = per > 0 ? (int)(((unsigned)nt * 37u) % (unsigned)per) : 0;
  auto clampc = [&](int x) {
    int y = min(x, per - 1) + rot;
    if (y >= per) y -= per;
    return c0 + y;
  };

  const bf16_t* wrow[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) wrow[i] = W + (size_t)min(n0 + i * 16 + l16, N - 1) * K + lg * 8;
  // NPC pieces per chunk: thread tid stages pieces tid + NTHR*q (< NPC; a
  // thread past the last piece loads a valid one and does not store it)
  const bf16_t* apiece[PPT];
  int aoff[PPT];
#pragma unroll
  for (int q = 0; q < PPT; ++q) {
    const int pc = min(tid + NTHR * q, NPC - 1), r = pc / PPR, cp = pc % PPR;
    apiece[q] = A + (size_t)min(m0 + r, M - 1) * lda + cp * 8;
    aoff[q] = r * ROWB + cp * 16;
  }
  const int boff = l16 * ROWB + lg * 16;  // this lane's A fragment within a 16-row block
  f32x4 acc[NR][MB];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A pieces travel as native vectors (a uint4 struct copy would become a
  // memcpy through private memory)
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  struct Stage {
    F8 w[U][NR];
    u32x4 a[PPT];
  };
  Stage S[NS];
  F8 B[2][U][MB];  // A fragments of the current and the next chunk
  // A pieces are issued before W so waiting for them does not wait for W
  auto gload = [&](Stage& st, int c) {
    const int k = c * U * GK;
#pragma unroll
    for (int q = 0; q < PPT; ++q) st.a[q] = *(const u32x4*)(apiece[q] + k);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < NR; ++i) st.w[u][i].u = *(const uint4*)(wrow[i] + k + u * GK);
  };
  auto stage = [&](int buf, const Stage& st) {
#pragma unroll
    for (int q = 0; q < PPT; ++q)
      if (NPC % NTHR == 0 || tid + NTHR * q < NPC) *(u32x4*)(lds + buf * BUFB + aoff[q]) = st.a[q];
  };
  auto readb = [&](F8 (&b)[U][MB], int buf) {
    const char* base = lds + buf * BUFB + boff;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < MB; ++j) b[u][j].u = *(const uint4*)(base + j * 16 * ROWB + u * GK * 2);
  };
  auto mfma = [&](const F8 (&b)[U][MB], const Stage& st) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(st.w[u][i].v, b[u][j].v, acc[i][j], 0, 0, 0);
  };
  // Chunk c0 + x: W and A pieces in register stage x % NS, A staged in LDS
  // buffer x % 3 at step x - 2 and read into B[x & 1] at step x - 1.  per
  // depends on blockIdx only, so every branch and barrier below is uniform
  // over the workgroup.  Loads past the last chunk are clamped (cache hits,
  // never multiplied).  Buffer (x + 2) % 3 is rewritten at step x; it was last
  // read at step x - 2, and two barriers separate the two.  sched_barrier keeps
  // each phase in program order (the scheduler would otherwise move W loads
  // ahead of A loads, and the in-order load counter would then make the LDS
  // store wait for W as well).
  if (per > 0) {
#pragma unroll
    for (int t = 0; t < NS; ++t) gload(S[t], clampc(t));
    stage(0, S[0]);
    if (per > 1) stage(1, S[1]);
    __syncthreads();
    readb(B[0], 0);
    // full groups first, with no conditions (branches would make the compiler's
    // wait counts conservative), then the last chunks with them
    auto step = [&](int x, auto tc, bool next, bool ahead) {
      constexpr int t = decltype(tc)::value;
      if (next) readb(B[(t + 1) & 1], (x + 1) % 3);
      __builtin_amdgcn_sched_barrier(0);
      mfma(B[t & 1], S[t]);
      __builtin_amdgcn_sched_barrier(0);
      gload(S[t], clampc(x + NS));
      __builtin_amdgcn_sched_barrier(0);
      if (ahead) stage((x + 2) % 3, S[(t + 2) % NS]);
      __syncthreads();
    };
    // NS steps per round, register stage t static in each (index_sequence unrolling)
    auto full_round = [&](int v, auto... ts) { (step(v + decltype(ts)::value, ts, true, true), ...); };
    auto last_round = [&](int v, auto... ts) {
      ((v + decltype(ts)::value < per ? step(v + decltype(ts)::value, ts, v + decltype(ts)::value + 1 < per,
                                             v + decltype(ts)::value + 2 < per)
                                      : void()),
       ...);
    };
    auto seq = [&](auto f, int v, auto is) {
      [&]<int... I>(std::integer_sequence<int, I...>) { f(v, std::integral_constant<int, I>{}...); }(is);
    };
    int v = 0;
    for (; v + NS + 1 < per; v += NS) seq(full_round, v, std::make_integer_sequence<int, NS>{});
    for (; v < per; v += NS) seq(last_round, v, std::make_integer_sequence<int, NS>{});
  }
  if constexpr (NR == 1 && (NWV == 4 || NWV == 3)) {
    if (rope) {
      rope_epilogue(acc, lds, w, n0, m0, M, e, l16, lg, rpos);
      return;
    }
  }
  store_tile<NR, MB>(acc, n0, m0, M, N, SK, ks, bz, e, sC, sR, A, part, l16, lg);
}

// 16 bytes per lane from sbase + off into LDS at lds + 16 * lane (gfx950
// global_load_lds_dwordx4; M0 holds the wave-uniform LDS address, one wait
// state after writing it).  Inline assembly: the compiler's own accounting of
// these loads would wait for all of them before any LDS read; the kernel waits
// for them itself (s_waitcnt vmcnt + barrier).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// Streaming kernel for every M (K % 64 == 0) with a ring of LDS chunk buffers.  Same
// tile ownership and accumulator layout as gemm_lds_kernel (NWV waves, each
// NR*16 W rows, 64 A rows, 16x16x32 products), but both operands travel
// global -> LDS by 16-byte direct loads: D chunks of 64 k (one 128-byte line
// of every W and A row) are in the ring, D - 1 of them in flight.  A product
// of this shape streams its weights once.  A CU's streaming rate stops growing
// once 2-3 chunks (about 40-70 KB) are in flight, while a deeper ring delays
// the first chunk (every workgroup's whole fill is queued at once), so the ring
// is 3-4 chunks deep rather than as deep as the LDS allows.  Each wave loads its own W rows;
// the 64 A rows of a chunk are split over the waves; one barrier per chunk
// makes the chunk visible and frees the buffer read in the previous step.  The
// 16-byte pieces of a row are permuted by (row / 2) mod 8 so the fragment reads
// of 16 consecutive rows fall in distinct banks.  Loads past the last chunk
// re-read it (cache hits, never multiplied), so every step waits for the same
// count.  grid (N tiles of NWV*NR*16 rows, m tiles * SK, batch).
template <int NR, int NWV, int D>
__global__ __launch_bounds__(NWV * 64) void gemm_dma_kernel(int M, int N, int K, const bf16_t* __restrict__ A,
                                                            int64_t lda, int64_t sA, const bf16_t* __restrict__ W,
                                                            int64_t sW, int SK, EpiArgs e, int64_t sC, int64_t sR,
                                                            float* __restrict__ part) {
  constexpr int MB = 4, TN = NR * 16;
  constexpr int KC = 2 * GK;               // k per chunk
  constexpr int ROWB = KC * 2;             // 128 bytes per row and chunk
  constexpr int AB = GM * ROWB;            // A bytes per chunk
  constexpr int WWB = TN * ROWB;           // W bytes per wave and chunk
  constexpr int CB = AB + NWV * WWB;       // one ring slot
  constexpr int AINS = AB / 1024;          // direct loads per A chunk (8 rows each)
  constexpr int AQ = (AINS + NWV - 1) / NWV;
  constexpr int WQ = WWB / 1024;
  constexpr int IPW = AQ + WQ;             // direct loads per wave and chunk
  constexpr bool SPARE = AQ * NWV != AINS;  // the surplus A loads land in a spare 1 KB
  static_assert(D >= 3 && (D - 2) * IPW <= 63, "wait count range");
  static_assert(D * CB + (SPARE ? 1024 : 0) <= 160 * 1024 && D * CB >= 16384, "LDS size");
  __shared__ __align__(16) char sm[D * CB + (SPARE ? 1024 : 0)];
  const int bz = blockIdx.z;
  const int nt = blockIdx.x;
  const int mt = blockIdx.y / SK;
  const int ks = blockIdx.y % SK;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  A += bz * sA;
  W += bz * sW;
  const bool rope = NR == 1 && (NWV == 4 || NWV == 3) && e.mode == EPI_QKV_ROPE;
  int n0 = (nt * NWV + w) * TN;
  if (rope) {
    if constexpr (NWV == 3) {
      const int pairs_per_head = e.Dh / 32;
      n0 = w < 2 ? (nt / pairs_per_head) * e.Dh + w * (e.Dh / 2) + (nt % pairs_per_head) * 16
                 : (e.Hq + e.Hkv) * e.Dh + nt * 16;
    } else {
      const int wg_per_head = e.Dh / 64, hd = nt / wg_per_head, sub = nt % wg_per_head;
      n0 = hd * e.Dh + (w & 1) * (e.Dh / 2) + (sub * 2 + (w >> 1)) * 16;
    }
  }
  const int m0 = mt * GM;
  // rotary rows' positions, loaded ahead of the product loop
  int rpos[4] = {0, 0, 0, 0};
  if (rope) rope_positions(e, m0, M, l16, rpos);
  const int nchunks = K / KC;
  const int c0 = (int)((int64_t)nchunks * ks / SK), c1 = (int)((int64_t)nchunks * (ks + 1) / SK);
  const int per = c1 - c0;
  // rotated k walk (see gemm_lds_kernel); fixed for a shape
  const int rot = per > 0 ? (int)(((unsigned)nt * 37u) % (unsigned)per) : 0;
  auto clampc = [&](int x) {
    int y = min(x, per - 1) + rot;
    if (y >= per) y -= per;
    return c0 + y;
  };
  auto pslot = [](int r) { return (r >> 1) & 7; };

  // direct-load source offsets (bytes from the chunk's first column): lane
  // writes LDS row lane / 8 of its instruction, slot lane % 8, which holds
  // piece slot ^ pslot(row) of that row
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)sm);
  const int drow = lane >> 3, dslot = lane & 7;
  uint32_t asrc[AQ], adst[AQ], wsrc[WQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int ins = w + NWV * q;
    const int r = (ins < AINS ? ins : 0) * 8 + drow;
    asrc[q] = (uint32_t)((int64_t)min(m0 + r, M - 1) * lda * 2 + ((dslot ^ pslot(r)) * 16));
    adst[q] = ins < AINS ? (uint32_t)(ins * 1024) : (uint32_t)(D * CB);
  }
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int r = q * 8 + drow;  // row within this wave's W rows
    wsrc[q] = (uint32_t)((int64_t)min(n0 + r, N - 1) * K * 2 + ((dslot ^ pslot(r)) * 16));
  }
  auto issue = [&](int x, int buf) __attribute__((always_inline)) {
    const int64_t kb = (int64_t)clampc(x) * ROWB;
    const char* ab = (const char*)A + kb;
    const char* wb = (const char*)W + kb;
    const uint32_t slot = lds0 + buf * CB;
#pragma unroll
    for (int q = 0; q < AQ; ++q) dma16(ab, asrc[q], adst[q] < (uint32_t)AB ? slot + adst[q] : lds0 + adst[q]);
#pragma unroll
    for (int q = 0; q < WQ; ++q) dma16(wb, wsrc[q], slot + AB + w * WWB + q * 1024);
  };
  // fragment read offsets (rows l16 of each 16-row block; pslot depends on l16 only)
  uint32_t frd[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) frd[s] = (uint32_t)(l16 * ROWB + (((s * 4 + lg) ^ pslot(l16)) * 16));

  f32x4 acc[NR][MB];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (per > 0) {
#pragma unroll
    for (int t = 0; t < D - 1; ++t) issue(t, t);
    int buf = 0;
    for (int x = 0; x < per; ++x) {
      // chunk x is complete once at most (D - 2) chunks' loads are outstanding
      // (vmcnt[3:0] and [15:14]; expcnt and lgkmcnt fields left at no-wait)
      constexpr int WN = (D - 2) * IPW;
      __builtin_amdgcn_s_waitcnt((WN & 0xf) | (0x7 << 4) | (0xf << 8) | (((WN >> 4) & 0x3) << 14));
      __syncthreads();
      issue(x + D - 1, buf == 0 ? D - 1 : buf - 1);
      const char* cb = sm + buf * CB;
      F8 wf[2][NR], af[2][MB];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < NR; ++i) wf[s][i].u = *(const uint4*)(cb + AB + w * WWB + i * 16 * ROWB + frd[s]);
#pragma unroll
        for (int j = 0; j < MB; ++j) af[s][j].u = *(const uint4*)(cb + j * 16 * ROWB + frd[s]);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
          for (int j = 0; j < MB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[s][i].v, af[s][j].v, acc[i][j], 0, 0, 0);
      buf = buf == D - 1 ? 0 : buf + 1;
    }
    // the re-reads past the last chunk land before the LDS is reused or freed
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));
  }
  if constexpr (NR == 1 && (NWV == 4 || NWV == 3)) {
    if (rope) {
      rope_epilogue(acc, sm, w, n0, m0, M, e, l16, lg, rpos);
      return;
    }
  }
  store_tile<NR, MB>(acc, n0, m0, M, N, SK, ks, bz, e, sC, sR, A, part, l16, lg);
}

// Sum split-K partials in split order and apply the epilogue.
// grid (ceil(Nout/256), M, batch)
template <typename T>
__global__ void splitk_reduce_kernel(int M, int N, int SK, const float* __restrict__ part, EpiArgs e, int64_t sC,
                                     int64_t sR, const T* __restrict__ A, int64_t sA) {
  const int m = blockIdx.y, bz = blockIdx.z;
  const int nout = blockIdx.x * blockDim.x + threadIdx.x;
  EpiArgs eb = e;
  eb.C = (char*)e.C + bz * sC * (e.mode == MEDUSA_EPI_F32 ? 4 : (int64_t)sizeof(T));
  if (e.R) eb.R = (const char*)e.R + bz * sR * (int64_t)sizeof(T);
  eb.A = A + bz * sA;
  const float* pp = part + ((size_t)bz * SK * M + m) * N;
  if (e.mode == MEDUSA_EPI_SWIGLU) {
    if (2 * nout + 1 >= N) return;
    float g = 0.f, u = 0.f;
    for (int s = 0; s < SK; ++s) {
      g += pp[(size_t)s * M * N + 2 * nout];
      u += pp[(size_t)s * M * N + 2 * nout + 1];
    }
    epi_swiglu<T>(eb, m, nout, g, u);
    return;
  }
  if (nout >= N) return;
  float v = 0.f;
  for (int s = 0; s < SK; ++s) v += pp[(size_t)s * M * N + nout];
  epi_store<T>(eb, m, nout, v);
}

struct GemmPlan {
  int SK, MB, NR, U, m_tiles, n_tiles;
  int NWV;   // gemm_lds_kernel: waves per workgroup (4, or 3 for 96-row tiles)
  bool KW;   // register kernel: the four waves split K
  bool LDS;  // 64-row activation tile: A staged in LDS (gemm_lds_kernel)
  bool DMA;  // ... both operands by direct loads into an LDS ring (gemm_dma_kernel)
  size_t part_bytes;
};

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return s ? atoi(s) : dflt;
}

// Tile shape, pipeline depth and K split for one product.  The MEDUSA_GEMM_*
// environment variables override the defaults for tuning runs only.
// Smallest M that takes the 64-row activation tile (gemm_lds_kernel /
// gemm_dma_kernel; rows past M re-read row M - 1): every M by default -- the
// direct-load kernel streams the weights faster than the register kernels
// even at M = 1 (Medusa heads at batch 1) -- or MEDUSA_GEMM_DMA_MIN_M (1..33,
// tuning runs; 33 sends M <= 32 to gemm_bf16_kernel).
int tile64_min_m() {
  static const int v = env_int("MEDUSA_GEMM_DMA_MIN_M", 1);
  return v < 1 ? 1 : (v > 33 ? 33 : v);
}

GemmPlan gemm_plan(int M, int N, int K, int batch) {
  static const int e_nr4 = env_int("MEDUSA_GEMM_NR4", 0);   // register kernel: 64 W rows per wave at M > 32
  static const int e_kw = env_int("MEDUSA_GEMM_KW", 1);     // register kernel: waves split K
  static const int e_lds = env_int("MEDUSA_GEMM_LDS", 1);   // 0: the register kernel for every M
  static const int e_lnr = env_int("MEDUSA_GEMM_LNR", 0);   // gemm_lds_kernel: W row blocks per wave (1 | 2)
  static const int e_u = env_int("MEDUSA_GEMM_U", 2);       // k-steps per chunk cap (1 | 2 | 4)
  static const int e_waves = env_int("MEDUSA_GEMM_WAVES", 1024);
  static const int e_sk = env_int("MEDUSA_GEMM_SK", 0);     // forced K split (0: from the wave target)
  static const int e_dma = env_int("MEDUSA_GEMM_DMA", 1);   // 64-row tiles on gemm_dma_kernel when the shape allows
  GemmPlan p;
  p.DMA = false;
  const int mrows = M < GM ? M : GM;
  p.MB = mrows <= 16 ? 1 : (mrows <= 32 ? 2 : 4);
  if (M >= tile64_min_m()) p.MB = 4;
  p.m_tiles = (M + GM - 1) / GM;
  p.LDS = p.MB == 4 && e_lds;
  p.KW = e_kw && !p.LDS;
  const int nsteps = K / GK;
  p.U = nsteps % 4 == 0 ? 4 : (nsteps % 2 == 0 ? 2 : 1);
  while (p.U > e_u && p.U > 1) p.U /= 2;
  if (p.LDS) {
    // two k-steps per chunk (four measured slower: more registers, same bytes in flight)
    p.U = nsteps % 2 == 0 ? 2 : 1;
    // One workgroup per CU streams best (a second one on some CUs leaves the
    // rest idle at the end): take 128-row tiles when they give >= 160
    // workgroups, else 64-row tiles, and split K across workgroups only when
    // even those leave most CUs idle.
    const int64_t per_tile = (int64_t)p.m_tiles * batch;
    const int64_t wg2 = (N + 127) / 128 * per_tile;
    p.NWV = 4;
    p.NR = e_lnr == 1 || e_lnr == 2 ? e_lnr : (wg2 >= 160 ? 2 : 1);
    if (!e_lnr && !e_sk) {
      // Workgroup tiles of 128, 96 or 64 rows: the kernel time follows the
      // rows per CU, so take the one with the fewest rows on the busiest CU
      // (ceil(workgroups / 256) * rows), the larger tile on a tie, among
      // shapes that give >= 160 workgroups (fewer take the K split below).
      // (waves, NR); 96-row tiles as 3 waves x 32 rows (measured faster than 6 x 16)
      const int cand[3][2] = {{4, 2}, {3, 2}, {4, 1}};
      int64_t best = -1;
      for (const auto& c : cand) {
        const int rows = c[0] * c[1] * 16;
        const int64_t wgs = (N + rows - 1) / rows * per_tile;
        if (wgs < 160) continue;
        const int64_t cost = (wgs + 255) / 256 * rows;
        if (best < 0 || cost < best) {
          best = cost;
          p.NWV = c[0];
          p.NR = c[1];
        }
      }
    }
    const int wg_rows = p.NWV * p.NR * 16;
    p.n_tiles = (N + wg_rows - 1) / wg_rows;
    const int64_t wgs = (int64_t)p.n_tiles * per_tile;
    int sk = e_sk > 0 ? e_sk : (wgs >= 160 ? 1 : (int)(256 / wgs));
    const int nchunks = nsteps / p.U;
    const int skmax = nchunks / 4 > 0 ? nchunks / 4 : 1;
    p.SK = sk < 1 ? 1 : (sk > skmax ? skmax : sk);
    // the direct loads address a row by a 32-bit byte offset from the chunk
    p.DMA = e_dma && p.U == 2 && (int64_t)N * K * 2 < ((int64_t)1 << 32);
  } else {
    p.NWV = 4;
    p.NR = p.MB == 4 && !e_nr4 ? 2 : 4;
    const int wg_rows = (p.KW ? 1 : 4) * p.NR * 16;
    p.n_tiles = (N + wg_rows - 1) / wg_rows;
    const int nchunks = nsteps / p.U;
    const int64_t waves = (int64_t)p.n_tiles * p.m_tiles * batch * 4;
    // aim at ~8 waves per CU while each wave keeps >= 2 chunks
    int sk = e_sk > 0 ? e_sk : (int)((e_waves + waves - 1) / waves);
    const int per_wg = p.KW ? 4 : 1;
    const int skmax = nchunks / (2 * per_wg) > 0 ? nchunks / (2 * per_wg) : 1;
    p.SK = sk < 1 ? 1 : (sk > skmax ? skmax : sk);
  }
  p.part_bytes = align_up((size_t)batch * p.SK * M * N * sizeof(float), 256);
  if (p.SK == 1) p.part_bytes = 0;
  return p;
}

// Launch the bf16 product kernel of plan p (partials, when left, go to ws).
void gemm_bf16_launch(const GemmPlan& p0, int M, int N, int K, const void* A, int64_t lda, int64_t strideA,
                      const void* W, int64_t strideW, const EpiArgs& e, int64_t strideC, int64_t strideR, void* ws,
                      int batch, hipStream_t stream) {
  // the direct loads address an activation row by a 32-bit byte offset too
  GemmPlan p = p0;
  if (p.DMA && (int64_t)M * lda * 2 >= ((int64_t)1 << 32)) p.DMA = false;
  dim3 grid(p.n_tiles, p.m_tiles * p.SK, batch);
#define GEMM_LAUNCH_KW(MBV, NRV, UV, KWV)                                                                      \
  hipLaunchKernelGGL((gemm_bf16_kernel<MBV, NRV, UV, KWV>), grid, dim3(GTHR), 0, stream, M, N, K, (const bf16_t*)A, \
                     lda, strideA, (const bf16_t*)W, strideW, p.SK, e, strideC, strideR, (float*)ws)
#define GEMM_LAUNCH(MBV, NRV, UV)              \
  do {                                         \
    if (p.KW) GEMM_LAUNCH_KW(MBV, NRV, UV, true); \
    else GEMM_LAUNCH_KW(MBV, NRV, UV, false);     \
  } while (0)
#define GEMM_LAUNCH_LDS(NRV, UV, NSV, NWVV)                                                                 \
  hipLaunchKernelGGL((gemm_lds_kernel<NRV, UV, NSV, NWVV>), grid, dim3(NWVV * 64), 0, stream, M, N, K,          \
                     (const bf16_t*)A, lda, strideA, (const bf16_t*)W, strideW, p.SK, e, strideC, strideR, (float*)ws)
#define GEMM_LAUNCH_DMA(NRV, NWVV, DV)                                                                       \
  hipLaunchKernelGGL((gemm_dma_kernel<NRV, NWVV, DV>), grid, dim3(NWVV * 64), 0, stream, M, N, K,               \
                     (const bf16_t*)A, lda, strideA, (const bf16_t*)W, strideW, p.SK, e, strideC, strideR, (float*)ws)
  // ring depth (64-k chunks): MEDUSA_GEMM_DMA_D = 3..6 overrides it for tuning runs
  static const int e_depth = env_int("MEDUSA_GEMM_DMA_D", 0);
  if (p.LDS && p.DMA) {
    const int kind = (p.NR - 1) * 2 + (p.NWV == 4 ? 1 : 0);
    // Measured on the 64-row projections and the 1-row heads: the first chunk
    // of a deep ring waits behind every workgroup's whole ring fill (about
    // 3.2 us for 10 chunks in flight, 1.9 us for 3), while the streaming rate
    // stays the same from 2-3 chunks in flight per CU on.
    static const int dflt[4] = {4, 4, 4, 3};  // (NR, waves) = (1, 3), (1, 4), (2, 3), (2, 4)
    const int dd = e_depth >= 3 && e_depth <= 6 ? e_depth : dflt[kind];
#define DMA_DEPTHS(NRV, NWVV)                    \
  do {                                           \
    if (dd == 3) GEMM_LAUNCH_DMA(NRV, NWVV, 3);  \
    else if (dd == 4) GEMM_LAUNCH_DMA(NRV, NWVV, 4); \
    else if (dd == 5) GEMM_LAUNCH_DMA(NRV, NWVV, 5); \
    else GEMM_LAUNCH_DMA(NRV, NWVV, 6);          \
  } while (0)
    if (kind == 0) DMA_DEPTHS(1, 3);
    else if (kind == 1) DMA_DEPTHS(1, 4);
    else if (kind == 2) DMA_DEPTHS(2, 3);
    else DMA_DEPTHS(2, 4);
#undef DMA_DEPTHS
  } else if (p.LDS) {
    if (p.NWV == 3 && p.NR == 1) {
      if (p.U == 2) GEMM_LAUNCH_LDS(1, 2, 4, 3);
      else GEMM_LAUNCH_LDS(1, 1, 4, 3);
    } else if (p.NWV == 3) {
      if (p.U == 2) GEMM_LAUNCH_LDS(2, 2, 4, 3);
      else GEMM_LAUNCH_LDS(2, 1, 4, 3);
    } else if (p.NR == 1) {
      if (p.U == 2) GEMM_LAUNCH_LDS(1, 2, 4, 4);
      else GEMM_LAUNCH_LDS(1, 1, 4, 4);
    } else {
      if (p.U == 2) GEMM_LAUNCH_LDS(2, 2, 4, 4);
      else GEMM_LAUNCH_LDS(2, 1, 4, 4);
    }
  } else if (p.MB == 1) {
    if (p.U == 4) GEMM_LAUNCH(1, 4, 4);
    else if (p.U == 2) GEMM_LAUNCH(1, 4, 2);
    else GEMM_LAUNCH(1, 4, 1);
  } else if (p.MB == 2) {
    if (p.U == 4) GEMM_LAUNCH(2, 4, 4);
    else if (p.U == 2) GEMM_LAUNCH(2, 4, 2);
    else GEMM_LAUNCH(2, 4, 1);
  } else if (p.NR == 2) {
    if (p.U == 4) GEMM_LAUNCH(4, 2, 4);
    else if (p.U == 2) GEMM_LAUNCH(4, 2, 2);
    else GEMM_LAUNCH(4, 2, 1);
  } else {
    if (p.U == 4) GEMM_LAUNCH(4, 4, 4);
    else if (p.U == 2) GEMM_LAUNCH(4, 4, 2);
    else GEMM_LAUNCH(4, 4, 1);
  }
#undef GEMM_LAUNCH
#undef GEMM_LAUNCH_KW
#undef GEMM_LAUNCH_LDS
#undef GEMM_LAUNCH_DMA
}

}  // namespace

extern "C" size_t medusa_gemm_workspace_size(int dtype, int M, int N, int K, int batch) {
  if (dtype != MEDUSA_BF16 || M <= 0 || N <= 0 || K <= 0 || batch <= 0 || K % GK) return 0;
  return gemm_plan(M, N, K, batch).part_bytes;
}

extern "C" int medusa_gemm(int dtype, int M, int N, int K, const void* A, int64_t lda, int64_t strideA, const void* W,
                           int64_t strideW, void* C, int64_t ldc, int64_t strideC, int batch, int epilogue,
                           const void* R, int64_t ldr, int64_t strideR, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  MEDUSA_REQUIRE(dtype_ok(dtype), MEDUSA_ERR_UNSUPPORTED, "gemm: dtype %d", dtype);
  MEDUSA_REQUIRE(M >= 0 && N > 0 && K > 0 && batch >= 1, MEDUSA_ERR_ARG, "gemm: bad sizes M=%d N=%d K=%d", M, N, K);
  MEDUSA_REQUIRE(epilogue >= MEDUSA_EPI_F32 && epilogue <= MEDUSA_EPI_SWIGLU, MEDUSA_ERR_ARG, "gemm: epilogue %d",
                 epilogue);
  MEDUSA_REQUIRE(epilogue != MEDUSA_EPI_RESID || R, MEDUSA_ERR_ARG, "gemm: residual epilogue needs R");
  MEDUSA_REQUIRE(epilogue != MEDUSA_EPI_SWIGLU || N % 2 == 0, MEDUSA_ERR_ARG, "gemm: SwiGLU needs even N");
  MEDUSA_REQUIRE(epilogue != MEDUSA_EPI_SILU_RESID_A || lda >= K, MEDUSA_ERR_ARG, "gemm: bad lda");
  MEDUSA_REQUIRE(lda >= K, MEDUSA_ERR_ARG, "gemm: lda < K");
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(A && W && C, MEDUSA_ERR_ARG, "gemm: null pointer");
  EpiArgs e{epilogue, C, ldc, R, ldr, A, lda, K, 0};
  if (dtype == MEDUSA_F32) {
    const int nout = epilogue == MEDUSA_EPI_SWIGLU ? N / 2 : N;
    dim3 grid((nout + 63) / 64, (M + 3) / 4, batch);
    hipLaunchKernelGGL(gemm_valu_kernel<float>, grid, dim3(64, 4), 0, stream, M, N, K, (const float*)A, lda, strideA,
                       (const float*)W, strideW, e, strideC, strideR);
    return check_launch("gemm fp32");
  }
  MEDUSA_REQUIRE(K % GK == 0, MEDUSA_ERR_UNSUPPORTED, "gemm: bf16 needs K %% 32 == 0 (K=%d)", K);
  MEDUSA_REQUIRE(lda % 8 == 0 && strideA % 8 == 0 && strideW % 8 == 0, MEDUSA_ERR_UNSUPPORTED,
                 "gemm: bf16 rows must be 16-byte aligned");
  // many rows: the square-tile kernel (compute-bound regime); MEDUSA_GEMM_TILE=0
  // keeps the streaming kernels for tuning runs
  static const int e_tile = env_int("MEDUSA_GEMM_TILE", 1);
  if (e_tile && gemm_tile_takes(M, N, K, epilogue))
    return gemm_tile_bf16(M, N, K, (const bf16_t*)A, lda, strideA, (const bf16_t*)W, strideW, epilogue, C, ldc,
                          strideC, (const bf16_t*)R, ldr, strideR, batch, stream);
  GemmPlan p = gemm_plan(M, N, K, batch);
  MEDUSA_REQUIRE(ws_bytes >= p.part_bytes && (p.SK == 1 || ws), MEDUSA_ERR_WORKSPACE, "gemm: workspace %zu < %zu",
                 ws_bytes, p.part_bytes);
  gemm_bf16_launch(p, M, N, K, A, lda, strideA, W, strideW, e, strideC, strideR, ws, batch, stream);
  int rc = check_launch("gemm bf16");
  if (rc) return rc;
  if (p.SK > 1) {
    const int nout = epilogue == MEDUSA_EPI_SWIGLU ? N / 2 : N;
    dim3 g2((nout + 255) / 256, M, batch);
    hipLaunchKernelGGL(splitk_reduce_kernel<bf16_t>, g2, dim3(256), 0, stream, M, N, p.SK, (const float*)ws, e,
                       strideC, strideR, (const bf16_t*)A, strideA);
    return check_launch("gemm split-K reduce");
  }
  return MEDUSA_OK;
}

// ---------------------------------------------------------------------------
// Residual add + RMSNorm fused with the product's split-K reduction
// ---------------------------------------------------------------------------
namespace {

// One 512-thread block per row; each thread holds NV vectors of 8 columns.
// SK > 0: acc = sum_s part[s][m][:] in split order, x[m,:] = bf16(x[m,:] + acc)
// is stored; SK == 0: x is only read.  Then y[m,:] = bf16(x[m,:] * inv * g)
// with inv = 1 / sqrt(mean(x[m,:]^2) + eps) taken over the stored bf16 x.
// The reads of x and g and of the partials are issued before their first use,
// the partials RN_SKB splits at a time, so a row costs ceil(SK / RN_SKB)
// memory round trips plus the block reduction (a loop that waited for each
// split's load before the next measured one round trip per split).
constexpr int RN_THREADS = 512;
constexpr int RN_SKB = 4;
template <int NV>
__global__ __launch_bounds__(RN_THREADS) void resid_rmsnorm_kernel(int M, int N, int SK,
                                                                   const float* __restrict__ part,
                                                                   bf16_t* __restrict__ x,
                                                                   const bf16_t* __restrict__ g, float eps,
                                                                   bf16_t* __restrict__ y) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int m = blockIdx.x, tid = threadIdx.x;
  bf16_t* xr = x + (size_t)m * N;
  u32x4 xraw[NV], graw[NV];
  float v[NV][8];
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int n = (q * RN_THREADS + tid) * 8;
    if (n < N) {
      xraw[q] = *(const u32x4*)(xr + n);
      graw[q] = *(const u32x4*)(g + n);
    }
  }
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int n = (q * RN_THREADS + tid) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[q][i] = 0.f;
    if (n >= N) continue;
    // RN_SKB splits per batch, all loads of a batch in flight together (a
    // tail batch re-reads the last split and leaves the copies out of the sum)
    for (int s0 = 0; s0 < SK; s0 += RN_SKB) {
      float4 a[RN_SKB], b[RN_SKB];
#pragma unroll
      for (int u = 0; u < RN_SKB; ++u) {
        const int sp = s0 + u < SK ? s0 + u : SK - 1;
        const float4* pp = (const float4*)(part + ((size_t)sp * M + m) * N + n);
        a[u] = pp[0];
        b[u] = pp[1];
      }
      // a select, not a branch, so that the loads stay ahead of every use
      // (adding +0 leaves a sum that started at +0 unchanged)
#pragma unroll
      for (int u = 0; u < RN_SKB; ++u) {
        const bool t = s0 + u < SK;
        v[q][0] += t ? a[u].x : 0.f; v[q][1] += t ? a[u].y : 0.f;
        v[q][2] += t ? a[u].z : 0.f; v[q][3] += t ? a[u].w : 0.f;
        v[q][4] += t ? b[u].x : 0.f; v[q][5] += t ? b[u].y : 0.f;
        v[q][6] += t ? b[u].z : 0.f; v[q][7] += t ? b[u].w : 0.f;
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int n = (q * RN_THREADS + tid) * 8;
    if (n >= N) continue;
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lo = __uint_as_float(xraw[q][i] << 16), hi = __uint_as_float(xraw[q][i] & 0xffff0000u);
      if (SK > 0) {
        const bf16_t blo = f32_to_bf16(lo + v[q][2 * i]), bhi = f32_to_bf16(hi + v[q][2 * i + 1]);
        lo = bf16_to_f32(blo);
        hi = bf16_to_f32(bhi);
        out[i] = (uint32_t)blo | ((uint32_t)bhi << 16);
      }
      v[q][2 * i] = lo;
      v[q][2 * i + 1] = hi;
      ss += lo * lo + hi * hi;
    }
    if (SK > 0) *(u32x4*)(xr + n) = out;
  }
  __shared__ float red[RN_THREADS / 64];
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < RN_THREADS / 64; ++i) tot += red[i];
  const float inv = 1.0f / sqrtf(tot / (float)N + eps);
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int n = (q * RN_THREADS + tid) * 8;
    if (n >= N) continue;
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g0 = __uint_as_float(graw[q][i] << 16), g1 = __uint_as_float(graw[q][i] & 0xffff0000u);
      out[i] = (uint32_t)f32_to_bf16(v[q][2 * i] * inv * g0) | ((uint32_t)f32_to_bf16(v[q][2 * i + 1] * inv * g1) << 16);
    }
    *(u32x4*)(y + (size_t)m * N + n) = out;
  }
}

}  // namespace

namespace medusa {

// bf16 RMSNorm rows of x (optionally after adding SK fp32 partials); N % 8 == 0, N <= 8192.
int resid_rmsnorm_bf16(int M, int N, int SK, const float* part, bf16_t* x, const bf16_t* g, float eps, bf16_t* y,
                       hipStream_t stream) {
  MEDUSA_REQUIRE(N % 8 == 0 && N <= 8192, MEDUSA_ERR_UNSUPPORTED, "rmsnorm bf16: N=%d (need N %% 8 == 0, <= 8192)", N);
  if (M == 0) return MEDUSA_OK;
  const int nv = (N + RN_THREADS * 8 - 1) / (RN_THREADS * 8);
  if (nv == 1)
    hipLaunchKernelGGL(resid_rmsnorm_kernel<1>, dim3(M), dim3(RN_THREADS), 0, stream, M, N, SK, part, x, g, eps, y);
  else
    hipLaunchKernelGGL(resid_rmsnorm_kernel<2>, dim3(M), dim3(RN_THREADS), 0, stream, M, N, SK, part, x, g, eps, y);
  return check_launch("resid_rmsnorm");
}

}  // namespace medusa

namespace medusa {

// Fused q/K/V projection with rotary embedding (bf16, M >= tile64_min_m(), Dh % 64 == 0):
// qkv = A W^T for W = [Hq q heads; Hkv k heads; Hkv v heads] x Dh rows, then
// q [B, T, Hq, Dh] and Kt [B, Hkv, T, Dh] rotated at pos[b*T + t], Vt as is.
// Returns MEDUSA_ERR_UNSUPPORTED (nothing launched) for shapes it does not take.
int gemm_qkv_rope_bf16(int B, int T, int K, int Hq, int Hkv, int Dh, const bf16_t* A, const bf16_t* W,
                       const int32_t* pos, const float* cos_t, const float* sin_t, int max_pos, bf16_t* q_out,
                       bf16_t* k_out, bf16_t* v_out, hipStream_t stream) {
  const int M = B * T, N = (Hq + 2 * Hkv) * Dh;
  if (M < tile64_min_m() || Dh % 64 || K % GK || K % 8) return MEDUSA_ERR_UNSUPPORTED;
  GemmPlan p = gemm_plan(M, N, K, 1);
  if (!p.LDS) return MEDUSA_ERR_UNSUPPORTED;
  p.NR = 1;
  p.NWV = 4;
  p.SK = 1;
  p.n_tiles = N / 64;
  // 48-row workgroups (a q or k rotary pair + one V block) when the pairs and
  // the V blocks come out even and that puts fewer rows on the busiest CU than
  // 64-row workgroups (MEDUSA_GEMM_QKV3 = 0 keeps 64 rows, for tuning runs)
  static const int e_qkv3 = env_int("MEDUSA_GEMM_QKV3", 1);
  const int pairs = (Hq + Hkv) * Dh / 32;
  if (e_qkv3 && pairs == Hkv * Dh / 16 && (pairs + 255) / 256 * 48 < (p.n_tiles + 255) / 256 * 64) {
    p.NWV = 3;
    p.n_tiles = pairs;
  }
  EpiArgs e{EPI_QKV_ROPE, nullptr, 0, nullptr, 0, A, K, K, 0, pos, cos_t, sin_t, max_pos, T, Hq, Hkv, Dh,
            q_out, k_out, v_out};
  gemm_bf16_launch(p, M, N, K, A, K, 0, W, 0, e, 0, 0, nullptr, 1, stream);
  return check_launch("gemm qkv rope");
}

}  // namespace medusa

extern "C" size_t medusa_gemm_resid_rmsnorm_workspace_size(int dtype, int M, int N, int K) {
  if (dtype != MEDUSA_BF16 || M <= 0 || N <= 0 || K <= 0 || K % GK) return 0;
  const GemmPlan p = gemm_plan(M, N, K, 1);
  return align_up((size_t)p.SK * M * N * sizeof(float), 256);
}

extern "C" int medusa_gemm_resid_rmsnorm(int dtype, int M, int N, int K, const void* A, int64_t lda, const void* W,
                                         void* X, const void* norm_w, float eps, void* Y, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
  MEDUSA_REQUIRE(dtype_ok(dtype), MEDUSA_ERR_UNSUPPORTED, "gemm_resid_rmsnorm: dtype %d", dtype);
  MEDUSA_REQUIRE(M >= 0 && N > 0 && K > 0 && lda >= K, MEDUSA_ERR_ARG, "gemm_resid_rmsnorm: bad sizes");
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(A && W && X && norm_w && Y, MEDUSA_ERR_ARG, "gemm_resid_rmsnorm: null pointer");
  if (dtype == MEDUSA_F32) {
    int rc = medusa_gemm(dtype, M, N, K, A, lda, 0, W, 0, X, N, 0, 1, MEDUSA_EPI_RESID, X, N, 0, nullptr, 0, stream);
    if (rc) return rc;
    return medusa_rmsnorm(dtype, M, N, X, norm_w, eps, Y, stream);
  }
  MEDUSA_REQUIRE(K % GK == 0 && lda % 8 == 0 && N % 8 == 0 && N <= 8192, MEDUSA_ERR_UNSUPPORTED,
                 "gemm_resid_rmsnorm: bf16 needs K %% 32 == 0, 16-byte rows, N %% 8 == 0 and N <= 8192");
  const GemmPlan p = gemm_plan(M, N, K, 1);
  const size_t need = align_up((size_t)p.SK * M * N * sizeof(float), 256);
  MEDUSA_REQUIRE(ws && ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "gemm_resid_rmsnorm: workspace %zu < %zu", ws_bytes,
                 need);
  EpiArgs e{MEDUSA_EPI_F32, nullptr, N, nullptr, 0, A, lda, K, 1};
  gemm_bf16_launch(p, M, N, K, A, lda, 0, W, 0, e, 0, 0, ws, 1, stream);
  int rc = check_launch("gemm_resid_rmsnorm product");
  if (rc) return rc;
  return resid_rmsnorm_bf16(M, N, p.SK, (const float*)ws, (bf16_t*)X, (const bf16_t*)norm_w, eps, (bf16_t*)Y, stream);
}
