// bf16 products C = A W^T with many rows (M >= 192): the compute-bound regime.
//
// With the Medusa heads applied to every tree node inside the verify forward
// (page "大模型推理 memory bandwidth bound (5) - Medusa", section 二.5: the heads
// run on all candidate positions in the same pass), the heads' products have
// M = batch * T rows (512 at batch 8, T 64), where each weight byte feeds 512
// rows and the matrix cores, not HBM, set the pace.  This kernel is the square
// tile design for that regime:
//
//  * a BM x 256 output tile per workgroup of 8 waves (2 along M x 4 along N),
//    each wave a (BM/2) x 64 block of v_mfma_f32_32x32x16_bf16 accumulators;
//    BM = 256, or 128 when 256-row tiles would leave most CUs idle;
//  * A and W chunks of 32 k go straight from global memory into LDS (16-byte
//    direct loads, global_load_lds_dwordx4), four chunks deep; rows keep K
//    contiguous (64 bytes a row), their four 16-byte pieces permuted by a
//    function of the row so the fragment reads of 32 consecutive rows fall in
//    distinct banks;
//  * one barrier per chunk, placed between its two 16-k steps, and fragments
//    always read one step ahead: a step's products run while the next step's
//    fragments (of the next chunk, across the barrier) come in from LDS;
//  * epilogues: fp32 store, dtype store, residual add, and the Medusa residual
//    A[m, n mod K] + SiLU(acc) (the head's h + SiLU(W1 h)).
// Rows of A past M and rows of W past N load a copy of the tile's last valid
// row; their outputs are never stored.
#include <stdlib.h>

#include <type_traits>

#include "common.h"
#include "medusa_model.h"

namespace medusa {
namespace {

constexpr int TBN = 256;             // output tile columns (W rows)
constexpr int TKC = 32;              // k per LDS chunk
constexpr int TNS = 4;               // chunks in LDS
constexpr int ROWB = TKC * 2;        // bytes per row of a chunk
constexpr int WTILEB = TBN * ROWB;   // bytes of one W chunk: 16 KB
constexpr int WNINS = WTILEB / 1024;  // 1 KB direct-load instructions per W chunk
constexpr int TTHR = 512;            // 8 waves
constexpr int NWV = TTHR / 64;

union Frag8 {
  uint4 u;
  bf16x8 v;
};

// piece c (16 bytes = 8 k) of row r sits in slot c ^ pslot(r)
__device__ __forceinline__ int pslot(int r) { return ((r >> 2) ^ (r >> 3)) & 3; }

// 16 bytes per lane from sbase + off into LDS at lds + 16 * lane (M0 = lds);
// one wait state between the M0 write and the load.  Inline assembly: the
// compiler's own accounting of these loads would wait for all of them before
// any LDS read; the kernel waits for them itself (s_waitcnt vmcnt + barrier).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16_t to_bf16(float x) {
  const __bf16 h = (__bf16)x;
  return __builtin_bit_cast(bf16_t, h);
}

struct TileEpi {
  int mode;
  void* C;
  int64_t ldc, sC;
  const bf16_t* R;
  int64_t ldr, sR;
  const bf16_t* A;  // MEDUSA_EPI_SILU_RESID_A: A[m, n mod K]
  int64_t lda, sA;
  int K;
};

// BM x TBN tile; waves 2 (M) x 4 (N), each a (BM/2) x 64 block of MB x NB
// accumulators
template <int BM>
__global__ __launch_bounds__(TTHR) void gemm_tile_kernel(int M, int N, int K, const bf16_t* __restrict__ A,
                                                          int64_t lda, int64_t sA, const bf16_t* __restrict__ W,
                                                          int64_t sW, TileEpi e) {
  constexpr int WM = 2, WN = 4;
  constexpr int MB = BM / WM / 32, NB = TBN / WN / 32;
  constexpr int ATILEB = BM * ROWB;      // bytes of one A chunk
  constexpr int ANINS = ATILEB / 1024;   // direct-load instructions per A chunk
  constexpr int AQ = ANINS / NWV, WQ = WNINS / NWV;  // ... issued by each wave
  constexpr int IPW = AQ + WQ;           // per wave and chunk
  constexpr int STB = ATILEB + WTILEB;   // bytes of one chunk (A then W) in LDS
  static_assert(AQ >= 1 && ANINS % NWV == 0 && WNINS % NWV == 0, "load split");
  // LDS: the TNS A chunks, then the TNS W chunks
  __shared__ __align__(16) char sm[TNS * STB];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = w / WN, wn = w % WN;  // wave block: rows wm*BM/WM.., columns wn*TBN/WN..
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * TBN, bz = blockIdx.z;
  A += bz * sA;
  W += bz * sW;
  const int nchunk = K / TKC;

  // ---- direct loads: instruction ii (0..NINS-1) of an A (W) chunk fills rows
  // ii*16 .. ii*16+15; this wave issues ii = w + NWV*q of both
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)sm);
  uint32_t aoff[AQ], woff[WQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int r = (w + NWV * q) * 16 + (lane >> 2);
    aoff[q] = (uint32_t)(min(r, M - 1 - m0) * lda * 2 + ((lane & 3) ^ pslot(r)) * 16);
  }
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int r = (w + NWV * q) * 16 + (lane >> 2);
    woff[q] = (uint32_t)(min(r, N - 1 - n0) * (int64_t)K * 2 + ((lane & 3) ^ pslot(r)) * 16);
  }
  auto issue = [&](int kc, int st) __attribute__((always_inline)) {
    const bf16_t* ab = A + (int64_t)m0 * lda + kc * TKC;
    const bf16_t* wb = W + (int64_t)n0 * K + kc * TKC;
    const uint32_t la = lds0 + st * ATILEB + w * 1024, lw = lds0 + TNS * ATILEB + st * WTILEB + w * 1024;
#pragma unroll
    for (int q = 0; q < AQ; ++q) dma16(ab, aoff[q], la + q * NWV * 1024);
#pragma unroll
    for (int q = 0; q < WQ; ++q) dma16(wb, woff[q], lw + q * NWV * 1024);
  };

  // ---- fragment offsets: A block mb (rows wm*MB*32 + mb*32 + lane%32), W
  // block nb (rows wn*NB*32 + nb*32 + lane%32), 16-k step s reads piece
  // 2s + lane/32
  uint32_t afr[MB][2], wfr[NB][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = wm * MB * 32 + mb * 32 + (lane & 31);
      afr[mb][s] = (uint32_t)(r * ROWB + (((2 * s + (lane >> 5)) ^ pslot(r)) * 16));
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int r = wn * NB * 32 + nb * 32 + (lane & 31);
      wfr[nb][s] = (uint32_t)(TNS * ATILEB + r * ROWB + (((2 * s + (lane >> 5)) ^ pslot(r)) * 16));
    }
  }

  f32x16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  Frag8 fa[2][MB], fw[2][NB];  // fragments of two 16-k steps
  auto read_frags = [&](int st, int s, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) fa[slot][mb].u = *(const uint4*)(sm + st * ATILEB + afr[mb][s]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) fw[slot][nb].u = *(const uint4*)(sm + st * WTILEB + wfr[nb][s]);
  };
  auto products = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][mb].v, fw[slot][nb].v, acc[mb][nb], 0, 0, 0);
  };

  // ---- pipeline.  Chunks 0 .. TNS-2 are in flight before the loop.  Chunk kc
  // (visible to every wave, its step-0 fragments already in slot 0) reads its
  // step-1 fragments, issues its step-0 products, then waits for this wave's
  // loads of chunk kc+1 and for the barrier (chunk kc+1 visible to all; every
  // wave done with chunk kc-1, whose buffer takes chunk kc-1+TNS), reads chunk
  // kc+1's step-0 fragments and issues its own step-1 products.  s_waitcnt
  // encoding: vmcnt[3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at
  // "no wait".
#pragma unroll
  for (int t = 0; t < TNS - 1; ++t)
    if (t < nchunk) issue(t, t);
  // the first chunk: wait for it everywhere, read its step-0 fragments
  if (nchunk - 1 >= TNS - 2) {
    constexpr int VN = (TNS - 2) * IPW;
    __builtin_amdgcn_s_waitcnt((VN & 0xf) | (0x7 << 4) | (0xf << 8) | (((VN >> 4) & 0x3) << 14));
  } else {
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));
  }
  __syncthreads();
  if (nchunk > 0) read_frags(0, 0, 0);
  for (int kc0 = 0; kc0 < nchunk; kc0 += TNS) {
    static_for<TNS>([&](auto UC) __attribute__((always_inline)) {
      constexpr int u = decltype(UC)::value;
      const int kc = kc0 + u;
      if (kc >= nchunk) return;
      read_frags(u, 1, 1);
      products(0);
      if (kc + 1 < nchunk) {
        // loads issued after chunk kc+1's: min(TNS-3, nchunk-2-kc) chunks
        if (nchunk - 2 - kc >= TNS - 3) {
          constexpr int VN = (TNS - 3) * IPW;
          __builtin_amdgcn_s_waitcnt((VN & 0xf) | (0x7 << 4) | (0xf << 8) | (((VN >> 4) & 0x3) << 14));
        } else {
          __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));
        }
        __syncthreads();
        if (kc - 1 + TNS < nchunk) issue(kc - 1 + TNS, (u + TNS - 1) % TNS);
        read_frags((u + 1) % TNS, 0, 0);
      }
      products(1);
    });
  }

  // ---- epilogue: lane holds column n = n0 + wn*NB*32 + nb*32 + lane%32 and
  // rows m = m0 + wm*MB*32 + mb*32 + 8j + 4*(lane/32) + i (acc[mb][nb][4j+i])
  auto store_all = [&](auto MODE) __attribute__((always_inline)) {
    constexpr int MD = decltype(MODE)::value;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = n0 + wn * NB * 32 + nb * 32 + (lane & 31);
      if (n >= N) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = m0 + wm * MB * 32 + mb * 32 + 8 * j + 4 * (lane >> 5) + i;
            if (m >= M) continue;
            const float v = acc[mb][nb][4 * j + i];
            const int64_t c = bz * e.sC + (int64_t)m * e.ldc + n;
            if constexpr (MD == MEDUSA_EPI_F32) {
              ((float*)e.C)[c] = v;
            } else if constexpr (MD == MEDUSA_EPI_STORE) {
              ((bf16_t*)e.C)[c] = to_bf16(v);
            } else if constexpr (MD == MEDUSA_EPI_RESID) {
              ((bf16_t*)e.C)[c] = to_bf16(bf16_to_f32(e.R[bz * e.sR + (int64_t)m * e.ldr + n]) + v);
            } else {
              const float r = bf16_to_f32(e.A[bz * e.sA + (int64_t)m * e.lda + (n % e.K)]);
              ((bf16_t*)e.C)[c] = to_bf16(r + silu(v));
            }
          }
    }
  };
  switch (e.mode) {
    case MEDUSA_EPI_F32: store_all(std::integral_constant<int, MEDUSA_EPI_F32>{}); break;
    case MEDUSA_EPI_STORE: store_all(std::integral_constant<int, MEDUSA_EPI_STORE>{}); break;
    case MEDUSA_EPI_RESID: store_all(std::integral_constant<int, MEDUSA_EPI_RESID>{}); break;
    default: store_all(std::integral_constant<int, MEDUSA_EPI_SILU_RESID_A>{}); break;
  }
}

}  // namespace

bool gemm_tile_takes(int M, int N, int K, int epilogue) {
  return M >= GEMM_TILE_MIN_M && epilogue != MEDUSA_EPI_SWIGLU && K % TKC == 0;
}

int gemm_tile_bf16(int M, int N, int K, const bf16_t* A, int64_t lda, int64_t strideA, const bf16_t* W,
                   int64_t strideW, int epilogue, void* C, int64_t ldc, int64_t strideC, const bf16_t* R, int64_t ldr,
                   int64_t strideR, int batch, hipStream_t stream) {
  MEDUSA_REQUIRE(gemm_tile_takes(M, N, K, epilogue), MEDUSA_ERR_UNSUPPORTED, "gemm tile: shape M=%d K=%d epi %d", M,
                 K, epilogue);
  // 32-bit per-lane load offsets: a tile's rows must span < 4 GB
  MEDUSA_REQUIRE((int64_t)256 * lda * 2 < (1ll << 31) && (int64_t)TBN * K * 2 < (1ll << 31), MEDUSA_ERR_UNSUPPORTED,
                 "gemm tile: rows too long");
  TileEpi e{epilogue, C, ldc, strideC, R, ldr, strideR, A, lda, strideA, K};
  // 256-row tiles unless they leave three quarters of the 256 CUs idle (the
  // 128-row tiles read twice the LDS bytes per product: slower per workgroup)
  const int64_t tiles256 = (int64_t)((M + 255) / 256) * ((N + TBN - 1) / TBN) * batch;
  if (tiles256 >= 64) {
    dim3 grid((M + 255) / 256, (N + TBN - 1) / TBN, batch);
    hipLaunchKernelGGL((gemm_tile_kernel<256>), grid, dim3(TTHR), 0, stream, M, N, K, A, lda, strideA, W, strideW, e);
  } else {
    dim3 grid((M + 127) / 128, (N + TBN - 1) / TBN, batch);
    hipLaunchKernelGGL((gemm_tile_kernel<128>), grid, dim3(TTHR), 0, stream, M, N, K, A, lda, strideA, W, strideW, e);
  }
  return check_launch("gemm tile");
}

}  // namespace medusa
