// Shared helpers of the libmedusa kernels and host entry points (gfx950 only).
#pragma once
#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string>

#include "medusa.h"

namespace medusa {

// ---- error reporting (thread-local message, status codes) ------------------
void set_error(const char* fmt, ...);
int fail(int code, const char* fmt, ...);
int check_launch(const char* what);

#define MEDUSA_REQUIRE(cond, code, ...)          \
  do {                                            \
    if (!(cond)) return ::medusa::fail(code, __VA_ARGS__); \
  } while (0)

#define MEDUSA_HIP(call)                                                           \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess)                                                          \
      return ::medusa::fail(MEDUSA_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

// ---- bfloat16 storage ------------------------------------------------------
typedef uint16_t bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}
// Round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

inline size_t dtype_size(int dtype) { return dtype == MEDUSA_BF16 ? 2 : 4; }
inline bool dtype_ok(int dtype) { return dtype == MEDUSA_F32 || dtype == MEDUSA_BF16; }

// Cross-lane butterfly without LDS: at step S a lane reads the value of its
// partner, which reads the lane's in turn.  Steps 0-3 are DPP permutations
// inside each row of 16 lanes (neighbours, pairs, mirror within 8, mirror
// within 16), step 4 pairs rows r and r ^ 1 and step 5 the two halves (the
// gfx950 v_permlane16/32_swap, which with both operands the same register
// return the lane's own value and its partner's).  Steps 0..4 combine the 32
// lanes of a half wave, 0..5 the whole wave; because partners are mutual, a
// commutative merge leaves the same result in every lane.
__device__ __forceinline__ unsigned lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
template <int S>
__device__ __forceinline__ unsigned bfly_u32(unsigned x) {
  if constexpr (S == 0) return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
  else if constexpr (S == 1) return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);
  else if constexpr (S == 2) return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);
  else if constexpr (S == 3) return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false);
  else if constexpr (S == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane_id() & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane_id() & 32) ? r[0] : r[1];
  }
}
template <int S>
__device__ __forceinline__ float bfly(float x) {
  return __uint_as_float(bfly_u32<S>(__float_as_uint(x)));
}
template <int S>
__device__ __forceinline__ int bfly(int x) {
  return (int)bfly_u32<S>((unsigned)x);
}
// f(std::integral_constant<int, S>{}) for S = 0 .. NSTEP-1 (6: a wave, 5: a half wave)
template <int NSTEP = 6, class F>
__device__ __forceinline__ void butterfly(F&& f) {
  f(std::integral_constant<int, 0>{});
  f(std::integral_constant<int, 1>{});
  f(std::integral_constant<int, 2>{});
  f(std::integral_constant<int, 3>{});
  f(std::integral_constant<int, 4>{});
  if constexpr (NSTEP > 5) f(std::integral_constant<int, 5>{});
}

__device__ __forceinline__ float wave_max(float v) {
  butterfly([&](auto S) { v = fmaxf(v, bfly<decltype(S)::value>(v)); });
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  butterfly([&](auto S) { v += bfly<decltype(S)::value>(v); });
  return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
  butterfly([&](auto S) { v = max(v, bfly<decltype(S)::value>(v)); });
  return v;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Embedding rows of tokens into x and their RMSNorm (weight w) into y in one
// launch; x as medusa_embed writes it, y by medusa_rmsnorm's formula
// (elementwise.hip).
int embed_rmsnorm(int dtype, int M, int d, const int32_t* tokens, const void* table, int V, const void* w, float eps,
                  void* x, void* y, hipStream_t stream);

// bf16 RMSNorm of M rows of length N (N % 8 == 0, N <= 8192, 16-byte aligned
// rows), optionally after adding SK fp32 split-K partials [SK][M][N] into x
// (gemm.hip).
int resid_rmsnorm_bf16(int M, int N, int SK, const float* part, bf16_t* x, const bf16_t* g, float eps, bf16_t* y,
                       hipStream_t stream);

// Fused q/K/V projection + rotary embedding for the bf16 verify forward
// (gemm.hip); MEDUSA_ERR_UNSUPPORTED without launching for shapes it does not
// take (Dh % 64 != 0, or M <= 32 under MEDUSA_GEMM_DMA_MIN_M = 33), in which
// case the caller runs medusa_gemm + medusa_rope_split.
int gemm_qkv_rope_bf16(int B, int T, int K, int Hq, int Hkv, int Dh, const bf16_t* A, const bf16_t* W,
                       const int32_t* pos, const float* cos_t, const float* sin_t, int max_pos, bf16_t* q_out,
                       bf16_t* k_out, bf16_t* v_out, hipStream_t stream);

// kv_compact with per-sequence stop (candidates_compact.hip): appends each
// sequence's accepted tokens up to and including the first stop_token (< 0:
// none) within its output and cache room, sets done[b] when it appends the stop
// token or fills a room, and leaves sequences with done[b] set untouched.
// Both compaction variants also write appended[b] (nullable): 1 when sequence b
// appended all a_b + 1 accepted tokens this step, else 0 (overflow, stop, done).
int kv_compact_stop(int dtype, const medusa_tree* t, int n_layers, int B, int Hkv, int Dh, int64_t Lmax, void* Kc,
                    void* Vc, const void* Kt, const void* Vt, const int32_t* best, const int32_t* accept_len,
                    int32_t* seq_len, const int32_t* tree_tokens, int32_t* out_tokens, int max_new, int32_t* n_out,
                    int32_t* done, int stop_token, int32_t* err_flag, int32_t* appended, hipStream_t stream);
int kv_compact_flags(int dtype, const medusa_tree* t, int n_layers, int B, int Hkv, int Dh, int64_t Lmax, void* Kc,
                     void* Vc, const void* Kt, const void* Vt, const int32_t* best, const int32_t* accept_len,
                     int32_t* seq_len, const int32_t* tree_tokens, int32_t* out_tokens, int max_new, int32_t* n_out,
                     int32_t* err_flag, int32_t* appended, hipStream_t stream);

// Square-tile bf16 product for many rows (gemm_tile.hip): M >= GEMM_TILE_MIN_M,
// K % 32 == 0, every epilogue but SwiGLU; W is [N, K] with K contiguous.
constexpr int GEMM_TILE_MIN_M = 192;
bool gemm_tile_takes(int M, int N, int K, int epilogue);
int gemm_tile_bf16(int M, int N, int K, const bf16_t* A, int64_t lda, int64_t strideA, const bf16_t* W,
                   int64_t strideW, int epilogue, void* C, int64_t ldc, int64_t strideC, const bf16_t* R, int64_t ldr,
                   int64_t strideR, int batch, hipStream_t stream);

}  // namespace medusa
