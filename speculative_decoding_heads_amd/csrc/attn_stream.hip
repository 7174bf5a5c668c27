// bf16 streaming tree attention (head size 64 or 128) on CDNA4 matrix cores.
//
// Computes, for every tree node i and query head h, softmax over the KV prefix
// plus the tree ancestors of i (page "大模型推理 memory bandwidth bound (5) -
// Medusa", section 一.2: a node only sees its predecessors; section 二.3: the
// prefix stays visible) times V.
//
// One workgroup of NW waves per (sequence, KV head, chunk of query rows, KV
// split).  The T*G query rows sharing a KV head (G = Hq/Hkv) are all served by
// a single pass over that head's keys, so K/V bytes are read from HBM once per
// KV head no matter how many query heads share them.  Wave w owns the
// 32-row block w (waves past the rows still help stream the tiles in):
//   * 64-key K and V tiles stream straight from HBM into LDS (16-byte direct
//     loads, no register staging), NBUF tiles deep, one barrier per tile;
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

// max / sum of a value and the one held by lane l ^ 32 (gfx950
// v_permlane32_swap: the two halves of the wave trade places without a trip
// through LDS, unlike a ds_bpermute shuffle)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 16-byte direct load per lane into LDS (gfx950 global_load_lds_dwordx4):
// lane l reads base + off and writes LDS at lds + 16 * l (M0 holds the
// wave-uniform LDS address, the SGPR pair the global base).  Written as inline
// assembly: the compiler's own bookkeeping of these loads waits for all of
// them before any LDS read, which would serialise the tile pipeline; the
// kernel waits for them itself (s_waitcnt vmcnt + barrier).  One wait state
// separates the M0 write from the load (the hazard the compiler's scheduler
// would otherwise cover).
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}

// LDS chunk permutation: 16-byte chunk c of key row k sits in slot c ^ swz(k)
template <int DH>
__device__ __forceinline__ int swz(int k) {
  if constexpr (DH == 128) return ((k & 3) << 2) | ((k >> 2) & 3);
  else return (k >> 1) & 7;
}

template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Tiles keep the cache layout in LDS (one 64-key tile of K, one of V, each
// DH*2 bytes a row; the NBUF K tiles first, then the NBUF V tiles), with the
// 16-byte chunks of a row permuted by swz so that the fragment reads fall in
// distinct banks.  K fragments are ds_read_b128 of one key row; the V^T operand
// of the P.V product is read with the gfx950 LDS transpose read
// (ds_read_b64_tr_b16): four lanes reading 32 contiguous bytes of one key row
// give each of 16 lanes four keys of one dimension.  Every lane's LDS read
// offsets are computed once; tiles that need no mask (all but a ragged last
// prefix tile and the tree tile, which come last) run with the buffer index a
// compile-time constant, so each read is one instruction with an immediate
// offset.  Rows past the valid keys of a tile load a copy of its first row
// (finite values that the mask then removes).
template <int DH, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void attn_lds_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc, int64_t Lmax,
    const int32_t* __restrict__ seq_len, const bf16_t* __restrict__ Kt, const bf16_t* __restrict__ Vt,
    const uint64_t* __restrict__ anc, int Tn, int Hq, int Hkv, int n_rchunks, float scale_log2, int n_splits,
    bf16_t* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  constexpr int ROWS_WG = NW * 32;
  constexpr int NKK = DH / 16;           // k-steps of the S^T product
  constexpr int NDB = DH / 32;           // 32-row blocks of O^T
  constexpr int CPR = DH / 8;            // 16-byte chunks per K/V row
  constexpr int ROWB = DH * 2;           // bytes per K/V row in LDS
  constexpr int TILEB = KT * ROWB;       // bytes of one K (or V) tile
  constexpr int RPI = 1024 / ROWB;       // rows per 64-lane load instruction
  constexpr int NI = KT / RPI;           // load instructions per K (or V) tile
  constexpr int MPH = NI / NW;           // ... of them issued by each wave
  constexpr int IPW = 2 * MPH;           // load instructions per wave and tile (K and V)
  static_assert(MPH >= 1 && NI % NW == 0, "tile load split");
  static_assert(NBUF >= 2 && (NBUF - 2) * IPW <= 63, "wait count range");
  static_assert(2 * NBUF * TILEB <= 160 * 1024, "LDS size");
  constexpr float RESCALE_SLACK = 8.0f;  // log2 units
  __shared__ __align__(16) char sm[2 * NBUF * TILEB];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z / n_rchunks;
  const int rchunk = blockIdx.z % n_rchunks;
  const int G = Hq / Hkv;
  const int R = Tn * G;
  const int r0 = rchunk * ROWS_WG;
  const int nr = min(ROWS_WG, R - r0);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hh = lane >> 5;

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
  // tiles 0 .. nfast-1 are whole prefix tiles; the rest (a ragged last prefix
  // tile, the tree tile) need the mask
  const int nfast = npre - (npre > 0 && t_end == tiles && (L % KT) != 0 ? 1 : 0);

  const size_t slab = (size_t)b * Hkv + kvh;
  const bf16_t* kc = Kc + slab * Lmax * DH;
  const bf16_t* vc = Vc + slab * Lmax * DH;
  const bf16_t* kt = Kt + slab * Tn * DH;
  const bf16_t* vt = Vt + slab * Tn * DH;
  const uint64_t tmask = Tn >= 64 ? ~0ull : ((1ull << Tn) - 1ull);

  // ---- this wave's row block: query row, node / head in group, mask word
  const bool act = w * 32 < nr;  // wave-uniform (w is)
  const int qrow = r0 + w * 32 + lq;
  const bool real = act && qrow < R;
  const int qnode = real ? qrow / G : 0;
  const int qg = real ? qrow % G : 0;
  const uint64_t qmask = real ? (anc[qnode] & tmask) : 1ull;
  bf16x8 qf[NKK];  // query fragments (B operand of S^T), loaded after the first tiles'
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  // ---- tile loads: instruction j of this wave fills rows (w + NW*j)*RPI ..
  // of a K tile and the same rows of a V tile; lane row / slot within it
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)sm);
  const int lrow = lane / CPR, lslot = lane % CPR;
  int drow[MPH];
  uint32_t doff[MPH];
#pragma unroll
  for (int j = 0; j < MPH; ++j) {
    drow[j] = (w + NW * j) * RPI + lrow;
    doff[j] = (uint32_t)(drow[j] * ROWB + ((lslot ^ swz<DH>(drow[j])) * 16));
  }
  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    const bool tree = t >= npre;
    const int64_t base = tree ? 0 : (int64_t)(t_begin + t) * KT;
    const int nvalid = tree ? Tn : (int)min<int64_t>(KT, L - base);
    const bf16_t* ksrc = tree ? kt : kc + base * DH;
    const bf16_t* vsrc = tree ? vt : vc + base * DH;
    const uint32_t lk = lds0 + buf * TILEB + w * 1024;
    if (nvalid >= KT) {
#pragma unroll
      for (int j = 0; j < MPH; ++j) {
        dma16(ksrc, doff[j], lk + NW * 1024 * j);
        dma16(vsrc, doff[j], lk + NW * 1024 * j + NBUF * TILEB);
      }
    } else {
#pragma unroll
      for (int j = 0; j < MPH; ++j) {
        const uint32_t off = drow[j] < nvalid ? doff[j] : doff[j] - (uint32_t)(drow[j] * ROWB);
        dma16(ksrc, off, lk + NW * 1024 * j);
        dma16(vsrc, off, lk + NW * 1024 * j + NBUF * TILEB);
      }
    }
  };

  // ---- LDS read offsets of this lane, relative to the tile's K (V) buffer:
  // K fragment kk of key kb*32 + lq at kl[kk] + kb*32*ROWB; V^T (transpose
  // read) for key block kb, sub-block ksub at vl[rd][db] + (kb*32 + 16*ksub)*ROWB,
  // where source lane s of 16-lane group g points at key 8*rd + 4*(g>>1) + s/4,
  // dimension db*32 + 16*(g&1) + 4*(s%4) (vl includes the V region's offset)
  uint32_t kl[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kl[kk] = (uint32_t)(lq * ROWB + (((kk * 2 + hh) ^ swz<DH>(lq)) * 16));
  uint32_t vl[2][NDB];
  {
    const int vg = lane >> 4, vs = lane & 15;
    const int vkey = 4 * (vg >> 1) + (vs >> 2);
    const int vdim = 16 * (vg & 1) + 4 * (vs & 3);
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int key = 8 * rd + vkey;
        const int dim = db * 32 + vdim;
        vl[rd][db] = (uint32_t)(NBUF * TILEB + key * ROWB + (((dim >> 3) ^ swz<DH>(key)) * 16) + (dim & 7) * 2);
      }
  }
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  union VF {
    v4i16 h[2];
    bf16x8 v;
  };

  // ---- one tile = two 32-key units.  K fragments, V^T fragments, S blocks and
  // P fragments live across the steps below (the next tile's unit-0 K
  // fragments are read before this tile's last unit is finished).
  Frag8 kf[NKK];
  VF vf[2][NDB];
  f32x16 s0, s1;
  bf16x8 pb[2];
  float mt1 = 0.f;
  // buffer byte offset: compile-time constant UB, or -1 for the runtime buf
  auto boff_of = [&](auto UB, int buf_rt) __attribute__((always_inline)) {
    constexpr int UBV = decltype(UB)::value;
    return UBV >= 0 ? (uint32_t)(UBV * TILEB) : (uint32_t)(buf_rt * TILEB);
  };
  auto load_k = [&](uint32_t boff, int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kf[kk].u = *(const uint4*)(sm + boff + kl[kk] + kb * 32 * ROWB);
  };
  auto load_v = [&](uint32_t boff, int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int ksub = 0; ksub < 2; ++ksub)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          vf[ksub][db].h[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(sm + boff + vl[rd][db] + (kb * 32 + 16 * ksub) * ROWB));
  };
  // S^T block: lane holds keys kb*32 + 8j + 4*hh + i (value s[4j+i]) of query
  // row lq (one accumulation chain: back-to-back dependent products issue at
  // full rate)
  auto qk = [&](f32x16& sr) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sr[e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) sr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk].v, qf[kk], sr, 0, 0, 0);
  };
  // masked keys -> -inf (MK: ragged prefix tile by key index, tree tile by the
  // ancestor word), then the row maximum in log2 units
  auto rowmax = [&](auto MASKED, f32x16& sr, int it, int kb) __attribute__((always_inline)) {
    if constexpr (decltype(MASKED)::value) {
      const bool tree = it >= npre;
      const int64_t base = tree ? 0 : (int64_t)(t_begin + it) * KT;
      const int nvalid = tree ? Tn : (int)min<int64_t>(KT, L - base);
      const int nv = nvalid - kb * 32;
      const uint32_t kbits = tree ? (uint32_t)(qmask >> (kb * 32))
                                  : (nv >= 32 ? 0xffffffffu : (nv <= 0 ? 0u : ((1u << nv) - 1u)));
      const uint32_t mine = kbits >> (4 * hh);
#pragma unroll
      for (int e = 0; e < 16; ++e) sr[e] = ((mine >> (8 * (e >> 2) + (e & 3))) & 1u) ? sr[e] : -INFINITY;
    }
    float mx = sr[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sr[e]);
    return halves_max(mx) * scale_log2;
  };
  // Rescales are rare once the running maxima settle, but each lane holds its own
  // row, so a per-lane branch would be if-converted into 64 multiplies (and an
  // exponential) on every unit.  A wave-wide vote skips the whole block unless
  // some lane needs it; lanes that do not keep a factor of 1.
  auto rescale = [&](float mt) __attribute__((always_inline)) {
    const bool need = mt > mrun + RESCALE_SLACK;
    if (__builtin_amdgcn_ballot_w64(need) == 0) return;
    const float alpha = need ? __builtin_amdgcn_exp2f(mrun - mt) : 1.0f;
    lrun *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
    mrun = need ? mt : mrun;
  };
  // P^T B operand: k-slot t of lane half hh <-> key 16*ksub + 8*(t/4) + 4*hh + t%4,
  // the same key order as the transposed V^T fragment.  The row sum is a
  // pairwise tree (independent adds rather than one dependent chain).
  auto expo = [&](const f32x16& sr) __attribute__((always_inline)) {
    const float negm = mrun == -INFINITY ? 0.f : -mrun;
    float p[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sr[e], scale_log2, negm));
    float t8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t8[e] = p[2 * e] + p[2 * e + 1];
    lrun += ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
    pb[0] = pack8(p);
    pb[1] = pack8(p + 8);
  };
  auto pv = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ksub = 0; ksub < 2; ++ksub)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ksub][db].v, pb[ksub], o[db], 0, 0, 0);
  };
  // First part of tile it (its unit-0 K fragments already in kf): unit 0's
  // products, unit 1's products beside unit 0's exponentials, unit 0's P.V
  // beside unit 1's row maximum, and unit 1's V^T fragments.
  auto head = [&](auto MASKED, uint32_t boff, int it) __attribute__((always_inline)) {
    qk(s0);
    load_k(boff, 1);
    load_v(boff, 0);
    rescale(rowmax(MASKED, s0, it, 0));
    qk(s1);
    expo(s0);
    pv();
    mt1 = rowmax(MASKED, s1, it, 1);
#pragma unroll
    for (int i = 0; i < NKK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // vector ALU
    }
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
    load_v(boff, 1);
  };
  // Rest of tile it: unit 1's exponentials and P.V.
  auto tail = [&]() __attribute__((always_inline)) {
    rescale(mt1);
    expo(s1);
    pv();
  };

  // ---- pipeline.  All NBUF buffers hold tiles: the one being computed and up
  // to NBUF-1 in flight.  In the middle of tile it (after its last LDS read)
  // each wave waits for its loads of tile it+1 and for its own LDS reads, the
  // barrier makes tile it+1 visible to all and frees tile it's buffer (every
  // wave has read what it needs of it), which is refilled with tile it+NBUF;
  // tile it+1's unit-0 K fragments are then read while tile it's last unit is
  // computed.  s_waitcnt encoding: vmcnt[3:0] and [15:14], expcnt [6:4],
  // lgkmcnt [11:8] (all-ones fields: no wait).
  auto mid = [&](int it, uint32_t boff_next) __attribute__((always_inline)) {
    if (it + 1 >= ntile) return;
    // loads issued after tile it+1's: min(NBUF-2, ntile-2-it) tiles
    if (ntile - 2 - it >= NBUF - 2) {
      constexpr int WN = (NBUF - 2) * IPW;
      __builtin_amdgcn_s_waitcnt((WN & 0xf) | (0x7 << 4) | (0x0 << 8) | (((WN >> 4) & 0x3) << 14));
    } else {
      __builtin_amdgcn_s_waitcnt(0x7 << 4);
    }
    __syncthreads();
    if (it + NBUF < ntile) issue_tile(it + NBUF, it % NBUF);
    if (act) load_k(boff_next, 0);
  };

  // prologue: tiles 0 .. NBUF-2, the query fragments, then tile NBUF-1
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < ntile) issue_tile(t, t);
  {
    // rows past R read row 0 of the head (in bounds); their columns of S and
    // O are never stored, so no select is needed (a select per load makes the
    // compiler serialise the loads on shared registers)
    const bf16_t* qp = q + (((size_t)b * Tn + qnode) * Hq + (size_t)kvh * G + qg) * DH;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      Frag8 f;
      f.u = *(const uint4*)(qp + kk * 16 + hh * 8);
      qf[kk] = f.v;
    }
  }
  // The query loads complete here, before the tile loop: the compiler counts
  // only its own loads, and its wait for these, were it placed inside the
  // loop, would also wait for every tile load issued after them.  The empty
  // asm reads each fragment, so the loads cannot sink past this point and that
  // wait lands here; it also covers the tile loads issued before them, so
  // after the barrier below tile 0 is visible to every wave.
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qf[kk]));
  if (NBUF - 1 < ntile) issue_tile(NBUF - 1, NBUF - 1);
  __syncthreads();
  if (act && ntile > 0) load_k(0, 0);

  // whole prefix tiles with the buffer a compile-time constant, then the
  // masked ones (ragged last prefix tile, tree tile) with a runtime buffer
  for (int it0 = 0; it0 < nfast; it0 += NBUF) {
    static_for<NBUF>([&](auto UC) __attribute__((always_inline)) {
      constexpr int u = decltype(UC)::value;
      const int it = it0 + u;
      if (it >= nfast) return;
      if (act) head(std::false_type{}, boff_of(UC, 0), it);
      mid(it, boff_of(std::integral_constant<int, (u + 1) % NBUF>{}, 0));
      if (act) tail();
    });
  }
  for (int it = nfast; it < ntile; ++it) {
    const std::integral_constant<int, -1> rt{};
    if (act) head(std::true_type{}, boff_of(rt, it % NBUF), it);
    mid(it, boff_of(rt, (it + 1) % NBUF));
    if (act) tail();
  }

  // ---- epilogue: O^T lane layout is rows dh = db*32 + 8j + 4*hh + i of query lq
  if (!real) return;
  const float ltot = halves_sum(lrun);
  if (n_splits == 1) {
    bf16_t* op = out + (((size_t)b * Tn + qnode) * Hq + (size_t)kvh * G + qg) * DH;
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 pk;  // round to nearest even (v_cvt_pk_bf16_f32)
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = (__bf16)(o[db][4 * j + i] * inv);
        *(bf16x4*)(op + db * 32 + 8 * j + 4 * hh) = pk;
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

// Waves per workgroup: 8 (the waves past the rows of a KV head still stream
// tiles in, which keeps more loads in flight); MEDUSA_ATTN_WAVES = 2 | 4 | 8
// forces a width for tuning runs.
int attn_stream_waves_forced() {
  static const int forced = [] {
    const char* e = getenv("MEDUSA_ATTN_WAVES");
    const int v = e ? atoi(e) : 0;
    return v == 2 || v == 4 || v == 8 ? v : 0;
  }();
  return forced;
}

template <int NW, int NBUF>
static void launch_d(int Dh, dim3 grid, hipStream_t stream, const bf16_t* q, const bf16_t* Kc, const bf16_t* Vc,
                     int64_t Lmax, const int32_t* seq_len, const bf16_t* Kt, const bf16_t* Vt, const uint64_t* anc,
                     int T, int Hq, int Hkv, int n_rchunks, float scale_log2, int n_splits, bf16_t* out, float* ws_o,
                     float* ws_ml) {
  if (Dh == 128)
    hipLaunchKernelGGL((attn_lds_kernel<128, NW, NBUF>), grid, dim3(NW * 64), 0, stream, q, Kc, Vc, Lmax, seq_len,
                       Kt, Vt, anc, T, Hq, Hkv, n_rchunks, scale_log2, n_splits, out, ws_o, ws_ml);
  else
    hipLaunchKernelGGL((attn_lds_kernel<64, NW, NBUF>), grid, dim3(NW * 64), 0, stream, q, Kc, Vc, Lmax, seq_len,
                       Kt, Vt, anc, T, Hq, Hkv, n_rchunks, scale_log2, n_splits, out, ws_o, ws_ml);
}

int launch_attn_stream(int Dh, int nw, dim3 grid, hipStream_t stream, const bf16_t* q, const bf16_t* Kc,
                       const bf16_t* Vc, int64_t Lmax, const int32_t* seq_len, const bf16_t* Kt, const bf16_t* Vt,
                       const uint64_t* anc, int T, int Hq, int Hkv, int n_rchunks, float scale_log2, int n_splits,
                       bf16_t* out, float* ws_o, float* ws_ml) {
  if (Dh != 128 && Dh != 64) return fail(MEDUSA_ERR_UNSUPPORTED, "tree_attention: streaming kernel takes Dh 64 or 128");
  // Tile depth: two buffers (one tile computed while the next streams in; a
  // deeper ring measured no faster and delays the first tile of short
  // per-workgroup runs).  MEDUSA_ATTN_NBUF = 2 | 3 | 4 forces a depth (tuning
  // runs).
  static const int forced_nbuf = [] {
    const char* e = getenv("MEDUSA_ATTN_NBUF");
    const int v = e ? atoi(e) : 0;
    return v == 2 || v == 3 || v == 4 ? v : 0;
  }();
  const int nbuf = forced_nbuf ? forced_nbuf : 2;
#define LD(NWV)                                                                                                      \
  do {                                                                                                               \
    if (nbuf == 2) launch_d<NWV, 2>(Dh, grid, stream, q, Kc, Vc, Lmax, seq_len, Kt, Vt, anc, T, Hq, Hkv, n_rchunks, \
                                    scale_log2, n_splits, out, ws_o, ws_ml);                                         \
    else if (nbuf == 4) launch_d<NWV, 4>(Dh, grid, stream, q, Kc, Vc, Lmax, seq_len, Kt, Vt, anc, T, Hq, Hkv,       \
                                         n_rchunks, scale_log2, n_splits, out, ws_o, ws_ml);                         \
    else launch_d<NWV, 3>(Dh, grid, stream, q, Kc, Vc, Lmax, seq_len, Kt, Vt, anc, T, Hq, Hkv, n_rchunks,           \
                          scale_log2, n_splits, out, ws_o, ws_ml);                                                   \
  } while (0)
  if (nw == 2) LD(2);
  else if (nw == 4) LD(4);
  else LD(8);
#undef LD
  return check_launch("tree_attention");
}

}  // namespace medusa
