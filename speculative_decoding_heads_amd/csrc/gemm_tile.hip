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
//  * A and W chunks of 64 k go straight from global memory into LDS (16-byte
//    direct loads, global_load_lds_dwordx4), two chunks deep for 256-row
//    tiles (128 KB of LDS) and three for 128-row tiles (144 KB: a third buffer
//    runs a product whose weights come from HBM 20% faster); a chunk holds a
//    whole 128-byte line of each row (chunks of 32 k fetched each line twice
//    through the vector L1 and ran 15-20% slower), the row's eight 16-byte
//    pieces permuted by a function of the row so the fragment reads of
//    consecutive rows fall in distinct banks;
//  * one barrier per chunk, before its last 16-k step: by then every wave
//    holds the chunk's fragments in registers, so its buffer takes the chunk
//    after next at once; fragments are always read one step ahead, so a
//    step's products run while the next step's fragments (of the next chunk,
//    across the barrier) come in from LDS;
//  * tiles ordered for the XCDs: the workgroups of one XCD take a contiguous
//    run of tiles, so those sharing a W tile share that XCD's L2;
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
constexpr int TTHR = 512;            // 8 waves
constexpr int NWV = TTHR / 64;

union Frag8 {
  uint4 u;
  bf16x8 v;
};

// LDS rows of ROWB bytes: piece c (16 bytes = 8 k) of row r sits in slot
// c ^ pslot(r).  The b128 reads of the fragments are served 16 lanes (16
// consecutive rows, one piece) at a time from 64 four-byte banks, i.e. by
// 256-byte windows: the permutation spreads those 16 rows over distinct
// 16-byte bank groups.
template <int ROWB>
__device__ __forceinline__ int pslot(int r) {
  if constexpr (ROWB == 64) return ((r >> 2) ^ (r >> 3)) & 3;  // 4 rows a window: slot from r/4
  else return (r >> 1) & 7;                                    // 2 rows a window: slot from r/2
}

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
// accumulators.  K advances KC at a time through NS LDS chunk buffers.
template <int BM, int KC, int NS>
__global__ __launch_bounds__(TTHR) void gemm_tile_kernel(int M, int N, int K, const bf16_t* __restrict__ A,
                                                          int64_t lda, int64_t sA, const bf16_t* __restrict__ W,
                                                          int64_t sW, TileEpi e) {
  constexpr int WM = 2, WN = 4;
  constexpr int MB = BM / WM / 32, NB = TBN / WN / 32;
  constexpr int ROWB = KC * 2;           // bytes of one row of a chunk
  constexpr int NPC = ROWB / 16;         // 16-byte pieces per row
  constexpr int RPI = 1024 / ROWB;       // rows per 1 KB direct-load instruction
  constexpr int SPC = KC / 16;           // 16-k MFMA steps per chunk
  constexpr int ATILEB = BM * ROWB;      // bytes of one A chunk
  constexpr int WTILEB = TBN * ROWB;     // bytes of one W chunk
  constexpr int ANINS = ATILEB / 1024, WNINS = WTILEB / 1024;  // direct loads per chunk
  constexpr int AQ = ANINS / NWV, WQ = WNINS / NWV;  // ... issued by each wave
  constexpr int IPW = AQ + WQ;           // per wave and chunk
  static_assert(AQ >= 1 && ANINS % NWV == 0 && WNINS % NWV == 0, "load split");
  static_assert(SPC % 2 == 0 && NS >= 2, "pipeline shape");
  // LDS: the NS A chunks, then the NS W chunks
  __shared__ __align__(16) char sm[NS * (ATILEB + WTILEB)];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = w / WN, wn = w % WN;  // wave block: rows wm*BM/WM.., columns wn*TBN/WN..
  // XCD-aware tile order.  Workgroups go to the 8 XCDs round robin by id, and
  // each XCD has its own L2: give XCD x a contiguous run of tile numbers, M
  // tiles fastest, so the workgroups that read one W tile (and neighbouring A
  // tiles) run side by side on one L2 instead of fetching W once per XCD.
  const int G = gridDim.x, L = blockIdx.x;
  const int xcd = L % 8, gq = G / 8, gr = G % 8;
  const int tile = xcd * gq + min(xcd, gr) + L / 8;
  const int nm = (M + BM - 1) / BM, nn = (N + TBN - 1) / TBN;
  const int m0 = (tile % nm) * BM, n0 = (tile / nm % nn) * TBN, bz = tile / nm / nn;
  A += bz * sA;
  W += bz * sW;
  const int nchunk = K / KC;

  // ---- direct loads: instruction ii (0..NINS-1) of an A (W) chunk fills rows
  // ii*RPI .. ii*RPI+RPI-1; this wave issues ii = w + NWV*q of both
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)sm);
  uint32_t aoff[AQ], woff[WQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int r = (w + NWV * q) * RPI + lane / NPC;
    aoff[q] = (uint32_t)(min(r, M - 1 - m0) * lda * 2 + ((lane % NPC) ^ pslot<ROWB>(r)) * 16);
  }
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int r = (w + NWV * q) * RPI + lane / NPC;
    woff[q] = (uint32_t)(min(r, N - 1 - n0) * (int64_t)K * 2 + ((lane % NPC) ^ pslot<ROWB>(r)) * 16);
  }
  auto issue = [&](int kc, int st) __attribute__((always_inline)) {
    const bf16_t* ab = A + (int64_t)m0 * lda + kc * KC;
    const bf16_t* wb = W + (int64_t)n0 * K + kc * KC;
    const uint32_t la = lds0 + st * ATILEB + w * 1024, lw = lds0 + NS * ATILEB + st * WTILEB + w * 1024;
#pragma unroll
    for (int q = 0; q < AQ; ++q) dma16(ab, aoff[q], la + q * NWV * 1024);
#pragma unroll
    for (int q = 0; q < WQ; ++q) dma16(wb, woff[q], lw + q * NWV * 1024);
  };

  // ---- fragment offsets: A block mb (rows wm*MB*32 + mb*32 + lane%32), W
  // block nb (rows wn*NB*32 + nb*32 + lane%32), 16-k step s reads piece
  // 2s + lane/32
  uint32_t afr[MB][SPC], wfr[NB][SPC];
#pragma unroll
  for (int s = 0; s < SPC; ++s) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = wm * MB * 32 + mb * 32 + (lane & 31);
      afr[mb][s] = (uint32_t)(r * ROWB + (((2 * s + (lane >> 5)) ^ pslot<ROWB>(r)) * 16));
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int r = wn * NB * 32 + nb * 32 + (lane & 31);
      wfr[nb][s] = (uint32_t)(NS * ATILEB + r * ROWB + (((2 * s + (lane >> 5)) ^ pslot<ROWB>(r)) * 16));
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
  // s_waitcnt vmcnt(n) lgkmcnt(0), expcnt at "no wait"; vmcnt sits in bits
  // [3:0] and [15:14].  lgkmcnt(0): this wave's fragment reads are done before
  // the barrier after which other waves overwrite the buffer they read.
  auto wait_loads = [](auto NV) __attribute__((always_inline)) {
    constexpr int n = decltype(NV)::value;
    __builtin_amdgcn_s_waitcnt((n & 0xf) | (0x7 << 4) | (((n >> 4) & 0x3) << 14));
  };

  // ---- pipeline.  Chunks 0 .. NS-1 are in flight before the loop.  Chunk kc
  // (visible to every wave, its step-0 fragments in slot 0) reads each next
  // step's fragments one step ahead of the products.  Before its last step
  // the wave waits for its own loads of chunk kc+1 and for the barrier: chunk
  // kc+1 is then visible to all, and every wave holds all of chunk kc's
  // fragments in registers (the barrier's fence waits for the LDS reads), so
  // chunk kc's buffer takes chunk kc+NS at once.  The last step's products
  // then run while chunk kc+1's step-0 fragments come in.
#pragma unroll
  for (int t = 0; t < NS; ++t)
    if (t < nchunk) issue(t, t);
  // the first chunk: wait for it everywhere, read its step-0 fragments
  if (nchunk >= NS) {
    wait_loads(std::integral_constant<int, (NS - 1) * IPW>{});
  } else {
    wait_loads(std::integral_constant<int, 0>{});
  }
  __syncthreads();
  if (nchunk > 0) read_frags(0, 0, 0);
  for (int kc0 = 0; kc0 < nchunk; kc0 += NS) {
    static_for<NS>([&](auto UC) __attribute__((always_inline)) {
      constexpr int u = decltype(UC)::value;
      const int kc = kc0 + u;
      if (kc >= nchunk) return;
      static_for<SPC - 1>([&](auto SC) __attribute__((always_inline)) {
        constexpr int st = decltype(SC)::value;
        read_frags(u, st + 1, (st + 1) & 1);
        // keep the reads ahead of the products: left to itself the scheduler
        // sinks them below the products to reuse the other slot's registers,
        // and the next products then wait for the LDS
        __builtin_amdgcn_sched_barrier(0);
        products(st & 1);
      });
      // loads issued after chunk kc+1's: chunks kc+2 .. min(kc+NS-1, nchunk-1)
      if (nchunk - 1 - kc >= NS) {
        wait_loads(std::integral_constant<int, (NS - 2) * IPW>{});
      } else {
        wait_loads(std::integral_constant<int, 0>{});
      }
      __syncthreads();
      if (kc + NS < nchunk) issue(kc + NS, u);
      // on the last chunk this reads a buffer no load targets any more, and
      // the fragments go unused: every path reaches the last products with the
      // same LDS reads in flight, so their wait covers only the fragments
      // read a step earlier
      read_frags((u + 1) % NS, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      products((SPC - 1) & 1);
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


// compute units of the current device (cached per device)
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

bool gemm_tile_takes(int M, int N, int K, int epilogue) {
  return M >= GEMM_TILE_MIN_M && epilogue != MEDUSA_EPI_SWIGLU && K % 64 == 0;
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
  const int64_t tiles256 = (int64_t)((M + 255) / 256) * ((N + TBN - 1) / TBN) * batch;
  const int64_t tiles128 = (int64_t)((M + 127) / 128) * ((N + TBN - 1) / TBN) * batch;
  MEDUSA_REQUIRE(tiles128 < (1ll << 31), MEDUSA_ERR_UNSUPPORTED, "gemm tile: too many tiles");
  // One workgroup per CU at a time (its LDS takes most of the CU's 160 KB),
  // so the time goes as the number of rounds of workgroups times the time of
  // one tile; a 128-row tile takes about 0.7 of a 256-row one (half the
  // products, but each W byte staged for half as many rows).
  const int64_t ncu = cu_count();
  const int64_t rounds256 = (tiles256 + ncu - 1) / ncu, rounds128 = (tiles128 + ncu - 1) / ncu;
  const bool bm256 = rounds128 * 7 >= rounds256 * 10;
  // k chunk of 64 (whole 128-byte lines of each row; two buffers at 256 rows,
  // three at 128) or of 32 (half lines, four buffers)
  static const bool kc32 = getenv("MEDUSA_TILE_KC") && atoi(getenv("MEDUSA_TILE_KC")) == 32;
  static const int bm_env = getenv("MEDUSA_TILE_BM") ? atoi(getenv("MEDUSA_TILE_BM")) : 0;
  if (bm_env == 256 || (bm_env != 128 && bm256)) {
    if (kc32)
      hipLaunchKernelGGL((gemm_tile_kernel<256, 32, 4>), dim3((unsigned)tiles256), dim3(TTHR), 0, stream, M, N, K, A,
                         lda, strideA, W, strideW, e);
    else
      hipLaunchKernelGGL((gemm_tile_kernel<256, 64, 2>), dim3((unsigned)tiles256), dim3(TTHR), 0, stream, M, N, K, A,
                         lda, strideA, W, strideW, e);
  } else {
    // three chunk buffers (MEDUSA_TILE_NS3 = 0: two, for tuning runs)
    static const bool ns3 = !(getenv("MEDUSA_TILE_NS3") && atoi(getenv("MEDUSA_TILE_NS3")) == 0);
    if (kc32)
      hipLaunchKernelGGL((gemm_tile_kernel<128, 32, 4>), dim3((unsigned)tiles128), dim3(TTHR), 0, stream, M, N, K, A,
                         lda, strideA, W, strideW, e);
    else if (ns3)
      hipLaunchKernelGGL((gemm_tile_kernel<128, 64, 3>), dim3((unsigned)tiles128), dim3(TTHR), 0, stream, M, N, K, A,
                         lda, strideA, W, strideW, e);
    else
      hipLaunchKernelGGL((gemm_tile_kernel<128, 64, 2>), dim3((unsigned)tiles128), dim3(TTHR), 0, stream, M, N, K, A,
                         lda, strideA, W, strideW, e);
  }
  return check_launch("gemm tile");
}

}  // namespace medusa
