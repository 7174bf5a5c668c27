// Dense products C = A W^T with fused epilogues, for the Medusa heads and the
// verify forward.
//
// The Medusa head of the page "大模型推理 memory bandwidth bound (5) - Medusa"
// (section 一.1) is z = SiLU(W1 h) + h followed by W2 z; the verify forward
// (section 二.5) runs the base model's projections on all T tree tokens at once.
// Both are weight-streaming products with few rows (M = batch or batch*T), so
// the bf16 kernel is built for HBM streaming, not for square tiles:
//
//  * bf16: a workgroup (4 waves) owns 64 rows of W and up to 64 rows of A over a
//    K range; W is the MFMA A-operand (16x16x32 bf16, fp32 accumulate) so each
//    lane loads 16 contiguous bytes of one W row per k-step, and the four waves
//    take interleaved k-steps of the range and are summed through LDS in a fixed
//    order.  When N/64 is too small to fill the chip, the K range is split
//    across workgroups and a second kernel adds the fp32 partials in a fixed
//    order and applies the epilogue.
//  * fp32: one thread per output with a sequential k loop, so a row's result
//    does not depend on M or on the row's position (plain decode and tree
//    verification agree bit for bit).
//
// Epilogues: store fp32; store in dtype; residual add; Medusa residual
// (A[m, n mod K] + SiLU(acc), the head's h + SiLU(W1 h) with W1 of size K x K);
// SwiGLU on row-interleaved gate/up weights (row 2j = gate j, row 2j+1 = up j).
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
};

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
constexpr int GN = 64;   // W rows per workgroup
constexpr int GM = 64;   // A rows per workgroup (max)
constexpr int GK = 32;   // k per MFMA step
constexpr int GTHR = 256;

union F8 {
  uint4 u;
  bf16x8 v;
};

// grid (N/64, ceil(M/64) * SK, batch).  MB = number of 16-row blocks of A used.
template <int MB>
__global__ __launch_bounds__(GTHR) void gemm_bf16_kernel(int M, int N, int K, const bf16_t* __restrict__ A, int64_t lda,
                                                         int64_t sA, const bf16_t* __restrict__ W, int64_t sW,
                                                         int SK, int ksteps_per_split, EpiArgs e, int64_t sC,
                                                         int64_t sR, float* __restrict__ part) {
  __shared__ float red[2][GN * GM];  // wave partial sums
  const int bz = blockIdx.z;
  const int nt = blockIdx.x;
  const int mt = blockIdx.y / SK;
  const int ks = blockIdx.y % SK;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  A += bz * sA;
  W += bz * sW;
  const int n0 = nt * GN, m0 = mt * GM;
  const int nsteps = K / GK;
  const int s_begin = ks * ksteps_per_split;
  const int s_end = min(s_begin + ksteps_per_split, nsteps);

  f32x4 acc[4][MB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // rows this lane feeds
  const bf16_t* wrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int n = n0 + i * 16 + l16;
    if (n >= N) n = N - 1;  // clamp (result discarded)
    wrow[i] = W + (size_t)n * K + lg * 8;
  }
  const bf16_t* arow[MB];
  bool avalid[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int m = m0 + j * 16 + l16;
    avalid[j] = m < M;
    arow[j] = A + (size_t)(avalid[j] ? m : 0) * lda + lg * 8;
  }

  constexpr int U = 4;  // k-steps in flight per wave
  int s = s_begin + w;
  for (; s + (U - 1) * 4 < s_end; s += U * 4) {
    F8 wf[U][4], af[U][MB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + u * 4) * GK;
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[u][i].u = *(const uint4*)(wrow[i] + k);
#pragma unroll
      for (int j = 0; j < MB; ++j) af[u][j].u = avalid[j] ? *(const uint4*)(arow[j] + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u][i].v, af[u][j].v, acc[i][j], 0, 0, 0);
  }
  for (; s < s_end; s += 4) {
    const int k = s * GK;
    F8 wf[4], af[MB];
#pragma unroll
    for (int i = 0; i < 4; ++i) wf[i].u = *(const uint4*)(wrow[i] + k);
#pragma unroll
    for (int j = 0; j < MB; ++j) af[j].u = avalid[j] ? *(const uint4*)(arow[j] + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < MB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i].v, af[j].v, acc[i][j], 0, 0, 0);
  }

  // fixed-order reduction of the 4 waves: (w2 -> w0, w3 -> w1), then (w1 -> w0)
  // C layout: acc[i][j][r] is W row n0 + 16i + 4*lg + r, A row m0 + 16j + l16.
  auto put = [&](int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < MB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[slot][(i * 16 + 4 * lg + r) * GM + j * 16 + l16] = acc[i][j][r];
  };
  auto add = [&](int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < MB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] += red[slot][(i * 16 + 4 * lg + r) * GM + j * 16 + l16];
  };
  if (w >= 2) put(w - 2);
  __syncthreads();
  if (w < 2) add(w);
  __syncthreads();
  if (w == 1) put(0);
  __syncthreads();
  if (w != 0) return;
  add(0);

  if (SK > 1) {
    // partials [batch][SK][M][N]
    float* pp = part + (((size_t)bz * SK + ks) * M) * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int m = m0 + j * 16 + l16;
        if (m >= M) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + i * 16 + 4 * lg + r;
          if (n < N) pp[(size_t)m * N + n] = acc[i][j][r];
        }
      }
    return;
  }
  EpiArgs eb = e;
  eb.C = (char*)e.C + bz * sC * (e.mode == MEDUSA_EPI_F32 ? 4 : 2);
  if (e.R) eb.R = (const char*)e.R + bz * sR * 2;
  eb.A = A;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int m = m0 + j * 16 + l16;
      if (m >= M) continue;
      const int nb = n0 + i * 16 + 4 * lg;
      if (e.mode == MEDUSA_EPI_SWIGLU) {
        if (nb + 1 < N) epi_swiglu<bf16_t>(eb, m, nb / 2, acc[i][j][0], acc[i][j][1]);
        if (nb + 3 < N) epi_swiglu<bf16_t>(eb, m, nb / 2 + 1, acc[i][j][2], acc[i][j][3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb + r < N) epi_store<bf16_t>(eb, m, nb + r, acc[i][j][r]);
      }
    }
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
  int SK, ksteps_per_split, m_tiles;
  size_t part_bytes;
};

GemmPlan gemm_plan(int M, int N, int K, int batch) {
  GemmPlan p;
  p.m_tiles = (M + GM - 1) / GM;
  const int n_tiles = (N + GN - 1) / GN;
  const int nsteps = K / GK;
  const int64_t wgs = (int64_t)n_tiles * p.m_tiles * batch;
  // fill ~512 workgroups; each split keeps >= 16 k-steps (4 per wave)
  int sk = (int)((512 + wgs - 1) / wgs);
  const int skmax = nsteps / 16 > 0 ? nsteps / 16 : 1;
  if (sk > skmax) sk = skmax;
  if (sk < 1) sk = 1;
  p.ksteps_per_split = (nsteps + sk - 1) / sk;
  p.ksteps_per_split = (p.ksteps_per_split + 3) / 4 * 4;  // whole wave rounds
  p.SK = (nsteps + p.ksteps_per_split - 1) / p.ksteps_per_split;
  p.part_bytes = p.SK > 1 ? align_up((size_t)batch * p.SK * M * N * sizeof(float), 256) : 0;
  return p;
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
  EpiArgs e{epilogue, C, ldc, R, ldr, A, lda, K};
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
  GemmPlan p = gemm_plan(M, N, K, batch);
  MEDUSA_REQUIRE(ws_bytes >= p.part_bytes && (p.SK == 1 || ws), MEDUSA_ERR_WORKSPACE, "gemm: workspace %zu < %zu",
                 ws_bytes, p.part_bytes);
  dim3 grid((N + GN - 1) / GN, p.m_tiles * p.SK, batch);
  const int mrows = M < GM ? M : GM;
  const int MB = (mrows + 15) / 16;
#define GEMM_LAUNCH(MBV)                                                                                          \
  hipLaunchKernelGGL(gemm_bf16_kernel<MBV>, grid, dim3(GTHR), 0, stream, M, N, K, (const bf16_t*)A, lda, strideA, \
                     (const bf16_t*)W, strideW, p.SK, p.ksteps_per_split, e, strideC, strideR, (float*)ws)
  if (MB <= 1) GEMM_LAUNCH(1);
  else if (MB == 2) GEMM_LAUNCH(2);
  else GEMM_LAUNCH(4);
#undef GEMM_LAUNCH
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
