// Launch interface of the bf16 streaming tree-attention kernel (attn_stream.hip).
#pragma once
#include "common.h"

namespace medusa {

constexpr int ATTN_KT = 64;  // keys per tile

// Waves per workgroup (32 query rows each) forced by MEDUSA_ATTN_WAVES (2, 4 or 8), else 0.
int attn_stream_waves_forced();

// nw waves per workgroup (2, 4 or 8); grid = (n_splits, Hkv, B * n_rchunks)
// with n_rchunks = ceil(R / (32 * nw)); ws_o / ws_ml used only when n_splits > 1.
int launch_attn_stream(int Dh, int nw, dim3 grid, hipStream_t stream, const bf16_t* q, const bf16_t* Kc,
                       const bf16_t* Vc, int64_t Lmax, const int32_t* seq_len, const bf16_t* Kt, const bf16_t* Vt,
                       const uint64_t* anc, int T, int Hq, int Hkv, int n_rchunks, float scale_log2, int n_splits,
                       bf16_t* out, float* ws_o, float* ws_ml);

}  // namespace medusa
