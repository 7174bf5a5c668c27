// Row-wise kernels of the verify forward: RMSNorm, rotary split of the fused
// Q/K/V projection into the query tensor and the tree K/V side buffers,
// embedding gather, row gather (the selected node's hidden state, which the
// page "大模型推理 memory bandwidth bound (5) - Medusa" hands to the next decode
// step's heads in section 二.7) and row argmax (the greedy root of section 二.4).
#include "common.h"
#include "medusa_model.h"

using namespace medusa;

namespace {

// one block (256 threads) per row
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(int N, const T* __restrict__ x, const T* __restrict__ w,
                                                      float eps, T* __restrict__ y) {
  const int m = blockIdx.x;
  const T* xr = x + (size_t)m * N;
  __shared__ float red[4];
  float ss = 0.f;
  for (int n = threadIdx.x; n < N; n += 256) {
    const float v = Elem<T>::load(xr, n);
    ss += v * v;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(tot / (float)N + eps);
  for (int n = threadIdx.x; n < N; n += 256)
    Elem<T>::store(y, (size_t)m * N + n, Elem<T>::load(xr, n) * inv * Elem<T>::load(w, n));
}

// grid (B*T, Hq + 2*Hkv), block Dh/2 threads (pairs i, i + Dh/2)
template <typename T>
__global__ void rope_split_kernel(int T_, int Hq, int Hkv, int Dh, const float* __restrict__ qkv,
                                  const int32_t* __restrict__ pos, const float* __restrict__ ct,
                                  const float* __restrict__ st, int max_pos, T* __restrict__ q_out, T* __restrict__ Kt,
                                  T* __restrict__ Vt) {
  const int row = blockIdx.x;  // b*T + t
  const int head = blockIdx.y;
  const int b = row / T_, t = row % T_;
  const int half = Dh / 2;
  const int W = (Hq + 2 * Hkv) * Dh;
  const float* src = qkv + (size_t)row * W + (size_t)head * Dh;
  int p = pos[row];
  p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const float x1 = src[i], x2 = src[i + half];
    if (head < Hq + Hkv) {
      const float c = ct[(size_t)p * half + i], s = st[(size_t)p * half + i];
      const float y1 = x1 * c - x2 * s;
      const float y2 = x2 * c + x1 * s;
      if (head < Hq) {
        T* d = q_out + ((size_t)row * Hq + head) * Dh;
        Elem<T>::store(d, i, y1);
        Elem<T>::store(d, i + half, y2);
      } else {
        const int h = head - Hq;
        T* d = Kt + (((size_t)b * Hkv + h) * T_ + t) * Dh;
        Elem<T>::store(d, i, y1);
        Elem<T>::store(d, i + half, y2);
      }
    } else {
      const int h = head - Hq - Hkv;
      T* d = Vt + (((size_t)b * Hkv + h) * T_ + t) * Dh;
      Elem<T>::store(d, i, x1);
      Elem<T>::store(d, i + half, x2);
    }
  }
}

template <typename T>
__global__ void embed_kernel(int d, const int32_t* __restrict__ tok, const T* __restrict__ table, int V,
                             T* __restrict__ out) {
  const int m = blockIdx.x;
  int v = tok[m];
  v = v < 0 ? 0 : (v >= V ? V - 1 : v);
  for (int n = threadIdx.x; n < d; n += blockDim.x) out[(size_t)m * d + n] = table[(size_t)v * d + n];
}

// Embedding gather fused with the first layer's input RMSNorm: one 256-thread
// block per row; with bf16 rows of d % 8 == 0 and d <= 8192 each thread keeps
// NV 16-byte pieces of the row in registers (one read of the table row), else
// element by element.  y = x * inv * w with inv = 1 / sqrt(mean(x^2) + eps),
// the formula of rmsnorm_kernel (the sum is taken in a different order).
template <typename T, int NV>
__global__ __launch_bounds__(256) void embed_rmsnorm_kernel(int d, const int32_t* __restrict__ tok,
                                                            const T* __restrict__ table, int V,
                                                            const T* __restrict__ w, float eps, T* __restrict__ x,
                                                            T* __restrict__ y) {
  const int m = blockIdx.x;
  int v = tok[m];
  v = v < 0 ? 0 : (v >= V ? V - 1 : v);
  const T* src = table + (size_t)v * d;
  T* xr = x + (size_t)m * d;
  T* yr = y + (size_t)m * d;
  __shared__ float red[4];
  float ss = 0.f;
  if constexpr (NV > 0) {
    // piece j of this thread: elements (j * 256 + tid) * 8 .. + 8
    uint4 raw[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e0 = (j * 256 + (int)threadIdx.x) * 8;
      if (e0 < d) {
        raw[j] = *(const uint4*)(src + e0);
        *(uint4*)(xr + e0) = raw[j];
        const uint32_t* u = (const uint32_t*)&raw[j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_to_f32((bf16_t)(u[q] & 0xffffu)), hi = bf16_to_f32((bf16_t)(u[q] >> 16));
          ss += lo * lo + hi * hi;
        }
      }
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = red[0] + red[1] + red[2] + red[3];
    const float inv = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e0 = (j * 256 + (int)threadIdx.x) * 8;
      if (e0 < d) {
        const uint4 wr = *(const uint4*)(w + e0);
        const uint32_t* u = (const uint32_t*)&raw[j];
        const uint32_t* g = (const uint32_t*)&wr;
        uint4 out;
        uint32_t* o = (uint32_t*)&out;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a0 = bf16_to_f32((bf16_t)(u[q] & 0xffffu)) * inv * bf16_to_f32((bf16_t)(g[q] & 0xffffu));
          const float a1 = bf16_to_f32((bf16_t)(u[q] >> 16)) * inv * bf16_to_f32((bf16_t)(g[q] >> 16));
          o[q] = (uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16);
        }
        *(uint4*)(yr + e0) = out;
      }
    }
  } else {
    for (int n = threadIdx.x; n < d; n += 256) {
      const T e = src[n];
      xr[n] = e;
      const float f = Elem<T>::load(&e, 0);
      ss += f * f;
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = red[0] + red[1] + red[2] + red[3];
    const float inv = 1.0f / sqrtf(tot / (float)d + eps);
    for (int n = threadIdx.x; n < d; n += 256) Elem<T>::store(yr, n, Elem<T>::load(src, n) * inv * Elem<T>::load(w, n));
  }
}

template <typename T>
__global__ void gather_rows_kernel(int T_, int d, const T* __restrict__ h, const int32_t* __restrict__ sel,
                                   T* __restrict__ out) {
  const int b = blockIdx.x;
  int s = sel[b];
  s = s < 0 ? 0 : (s >= T_ ? T_ - 1 : s);
  for (int n = threadIdx.x; n < d; n += blockDim.x) out[(size_t)b * d + n] = h[((size_t)b * T_ + s) * d + n];
}

__global__ __launch_bounds__(256) void argmax_rows_kernel(int V, const float* __restrict__ x, int64_t ldx,
                                                          int32_t* __restrict__ out) {
  const int m = blockIdx.x;
  const float* r = x + (size_t)m * ldx;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int k = threadIdx.x; k < V; k += 256) {
    const float v = r[k];
    if (v > bv) {
      bv = v;
      bi = k;
    }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  butterfly([&](auto S) {
    constexpr int s = decltype(S)::value;
    const float v2 = bfly<s>(bv);
    const int i2 = bfly<s>(bi);
    if (v2 > bv || (v2 == bv && i2 < bi)) {
      bv = v2;
      bi = i2;
    }
  });
  if ((threadIdx.x & 63) == 0) {
    sv[threadIdx.x >> 6] = bv;
    si[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int j = 1; j < 4; ++j)
      if (sv[j] > bv || (sv[j] == bv && si[j] < bi)) {
        bv = sv[j];
        bi = si[j];
      }
    out[m] = bi == 0x7fffffff ? 0 : bi;
  }
}

}  // namespace

extern "C" int medusa_rmsnorm(int dtype, int M, int N, const void* x, const void* w, float eps, void* y,
                              hipStream_t stream) {
  MEDUSA_REQUIRE(dtype_ok(dtype), MEDUSA_ERR_UNSUPPORTED, "rmsnorm: dtype");
  MEDUSA_REQUIRE(M >= 0 && N > 0, MEDUSA_ERR_ARG, "rmsnorm: bad sizes");
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(x && w && y, MEDUSA_ERR_ARG, "rmsnorm: null pointer");
  const bool vec_ok = N % 8 == 0 && N <= 8192 && (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) & 15) == 0;
  if (dtype == MEDUSA_BF16 && vec_ok)
    return resid_rmsnorm_bf16(M, N, 0, nullptr, (bf16_t*)x, (const bf16_t*)w, eps, (bf16_t*)y, stream);
  if (dtype == MEDUSA_F32)
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(M), dim3(256), 0, stream, N, (const float*)x, (const float*)w, eps,
                       (float*)y);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3(M), dim3(256), 0, stream, N, (const bf16_t*)x, (const bf16_t*)w,
                       eps, (bf16_t*)y);
  return check_launch("rmsnorm");
}

extern "C" int medusa_rope_split(int dtype, int B, int T, int Hq, int Hkv, int Dh, const float* qkv,
                                 const int32_t* pos, const float* cos_tab, const float* sin_tab, int max_pos,
                                 void* q_out, void* Kt, void* Vt, hipStream_t stream) {
  MEDUSA_REQUIRE(dtype_ok(dtype), MEDUSA_ERR_UNSUPPORTED, "rope_split: dtype");
  MEDUSA_REQUIRE(B >= 0 && T > 0 && Hq > 0 && Hkv > 0 && Dh > 0 && Dh % 2 == 0 && max_pos > 0, MEDUSA_ERR_ARG,
                 "rope_split: bad sizes");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(qkv && pos && cos_tab && sin_tab && q_out && Kt && Vt, MEDUSA_ERR_ARG, "rope_split: null pointer");
  dim3 grid(B * T, Hq + 2 * Hkv);
  const int thr = Dh / 2 < 64 ? 64 : (Dh / 2 > 256 ? 256 : Dh / 2);
  if (dtype == MEDUSA_F32)
    hipLaunchKernelGGL(rope_split_kernel<float>, grid, dim3(thr), 0, stream, T, Hq, Hkv, Dh, qkv, pos, cos_tab,
                       sin_tab, max_pos, (float*)q_out, (float*)Kt, (float*)Vt);
  else
    hipLaunchKernelGGL(rope_split_kernel<bf16_t>, grid, dim3(thr), 0, stream, T, Hq, Hkv, Dh, qkv, pos, cos_tab,
                       sin_tab, max_pos, (bf16_t*)q_out, (bf16_t*)Kt, (bf16_t*)Vt);
  return check_launch("rope_split");
}

extern "C" int medusa_embed(int dtype, int M, int d, const int32_t* tokens, const void* table, int V, void* out,
                            hipStream_t stream) {
  MEDUSA_REQUIRE(dtype_ok(dtype), MEDUSA_ERR_UNSUPPORTED, "embed: dtype");
  MEDUSA_REQUIRE(M >= 0 && d > 0 && V > 0, MEDUSA_ERR_ARG, "embed: bad sizes");
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(tokens && table && out, MEDUSA_ERR_ARG, "embed: null pointer");
  if (dtype == MEDUSA_F32)
    hipLaunchKernelGGL(embed_kernel<float>, dim3(M), dim3(256), 0, stream, d, tokens, (const float*)table, V,
                       (float*)out);
  else
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(M), dim3(256), 0, stream, d, tokens, (const bf16_t*)table, V,
                       (bf16_t*)out);
  return check_launch("embed");
}

namespace medusa {

int embed_rmsnorm(int dtype, int M, int d, const int32_t* tokens, const void* table, int V, const void* w, float eps,
                  void* x, void* y, hipStream_t stream) {
  MEDUSA_REQUIRE(dtype_ok(dtype), MEDUSA_ERR_UNSUPPORTED, "embed_rmsnorm: dtype");
  MEDUSA_REQUIRE(M >= 0 && d > 0 && V > 0, MEDUSA_ERR_ARG, "embed_rmsnorm: bad sizes");
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(tokens && table && w && x && y, MEDUSA_ERR_ARG, "embed_rmsnorm: null pointer");
  // 16-byte pieces need aligned rows: d % 8 == 0 and 16-byte aligned bases
  const bool vec = dtype == MEDUSA_BF16 && d % 8 == 0 && d <= 8192 &&
                   (((uintptr_t)table | (uintptr_t)w | (uintptr_t)x | (uintptr_t)y) & 15) == 0;
  if (dtype == MEDUSA_F32)
    hipLaunchKernelGGL((embed_rmsnorm_kernel<float, 0>), dim3(M), dim3(256), 0, stream, d, tokens,
                       (const float*)table, V, (const float*)w, eps, (float*)x, (float*)y);
  else if (!vec)
    hipLaunchKernelGGL((embed_rmsnorm_kernel<bf16_t, 0>), dim3(M), dim3(256), 0, stream, d, tokens,
                       (const bf16_t*)table, V, (const bf16_t*)w, eps, (bf16_t*)x, (bf16_t*)y);
  else if (d <= 2048)
    hipLaunchKernelGGL((embed_rmsnorm_kernel<bf16_t, 1>), dim3(M), dim3(256), 0, stream, d, tokens,
                       (const bf16_t*)table, V, (const bf16_t*)w, eps, (bf16_t*)x, (bf16_t*)y);
  else if (d <= 4096)
    hipLaunchKernelGGL((embed_rmsnorm_kernel<bf16_t, 2>), dim3(M), dim3(256), 0, stream, d, tokens,
                       (const bf16_t*)table, V, (const bf16_t*)w, eps, (bf16_t*)x, (bf16_t*)y);
  else
    hipLaunchKernelGGL((embed_rmsnorm_kernel<bf16_t, 4>), dim3(M), dim3(256), 0, stream, d, tokens,
                       (const bf16_t*)table, V, (const bf16_t*)w, eps, (bf16_t*)x, (bf16_t*)y);
  return check_launch("embed_rmsnorm");
}

}  // namespace medusa

extern "C" int medusa_gather_rows(int dtype, int B, int T, int d, const void* h, const int32_t* sel, void* out,
                                  hipStream_t stream) {
  MEDUSA_REQUIRE(dtype_ok(dtype), MEDUSA_ERR_UNSUPPORTED, "gather_rows: dtype");
  MEDUSA_REQUIRE(B >= 0 && T > 0 && d > 0, MEDUSA_ERR_ARG, "gather_rows: bad sizes");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(h && sel && out, MEDUSA_ERR_ARG, "gather_rows: null pointer");
  if (dtype == MEDUSA_F32)
    hipLaunchKernelGGL(gather_rows_kernel<float>, dim3(B), dim3(256), 0, stream, T, d, (const float*)h, sel,
                       (float*)out);
  else
    hipLaunchKernelGGL(gather_rows_kernel<bf16_t>, dim3(B), dim3(256), 0, stream, T, d, (const bf16_t*)h, sel,
                       (bf16_t*)out);
  return check_launch("gather_rows");
}

extern "C" int medusa_argmax_rows(int M, int V, const float* x, int64_t ldx, int32_t* out, hipStream_t stream) {
  MEDUSA_REQUIRE(M >= 0 && V > 0 && ldx >= V, MEDUSA_ERR_ARG, "argmax_rows: bad sizes");
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(x && out, MEDUSA_ERR_ARG, "argmax_rows: null pointer");
  hipLaunchKernelGGL(argmax_rows_kernel, dim3(M), dim3(256), 0, stream, V, x, ldx, out);
  return check_launch("argmax_rows");
}
