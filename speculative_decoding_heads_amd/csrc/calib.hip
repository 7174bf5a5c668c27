// Tree calibration: the static tree from per-(depth, rank) acceptance rates
// (host) and the teacher-forced hit counts of the heads (device).
//
// Page "大模型推理 memory bandwidth bound (5) - Medusa", section 一.2: the sparse
// tree is fixed ahead of time and keeps the probable candidate paths.  The
// page gives no construction; the reading taken here: a path's probability is
// the product of the per-(depth, rank) acceptance rates along it, the tree of
// n nodes keeps the n - 1 most probable paths, which maximises the expected
// accepted length under independent depths.
#include <math.h>

#include <queue>
#include <vector>

#include "common.h"

using namespace medusa;

namespace {

struct Cand {
  double p;
  std::vector<int32_t> path;
};

// pop order: higher probability, then shorter path, then smaller ranks
struct After {
  bool operator()(const Cand& a, const Cand& b) const {
    if (a.p != b.p) return a.p < b.p;
    if (a.path.size() != b.path.size()) return a.path.size() > b.path.size();
    return a.path > b.path;
  }
};

constexpr int HITS_THREADS = 256;
constexpr int HITS_MAX_BINS = 4096;

// grid over positions t (one thread per (t, head)); per-block LDS bins, then
// one 64-bit atomic per non-zero bin
__global__ __launch_bounds__(HITS_THREADS) void head_hits_kernel(int N, int H, int K, const int32_t* __restrict__ topk,
                                                                  const int32_t* __restrict__ tokens, int n_tokens,
                                                                  unsigned long long* __restrict__ counts,
                                                                  unsigned long long* __restrict__ positions) {
  __shared__ unsigned int bins[HITS_MAX_BINS];
  __shared__ unsigned int pbins[64];
  const int nb = H * K;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) bins[i] = 0;
  for (int i = threadIdx.x; i < H && i < 64; i += blockDim.x) pbins[i] = 0;
  __syncthreads();
  const int64_t pairs = (int64_t)N * H;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < pairs; e += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(e / H), k = (int)(e % H);
    const int64_t j = (int64_t)t + k + 2;
    if (j >= n_tokens) continue;
    const int32_t target = tokens[j];
    const int32_t* row = topk + e * K;
    if (k < 64) atomicAdd(&pbins[k], 1u);
    else atomicAdd(positions + k, 1ull);
    for (int r = 0; r < K; ++r)
      if (row[r] == target) atomicAdd(&bins[k * K + r], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += blockDim.x)
    if (bins[i]) atomicAdd(counts + i, (unsigned long long)bins[i]);
  for (int i = threadIdx.x; i < H && i < 64; i += blockDim.x)
    if (pbins[i]) atomicAdd(positions + i, (unsigned long long)pbins[i]);
}

}  // namespace

extern "C" int medusa_tree_from_acceptance(const double* acc, int32_t H, int32_t K, int32_t n_nodes, int32_t* ranks,
                                           int32_t* offsets, double* expected) {
  MEDUSA_REQUIRE(acc && ranks && offsets, MEDUSA_ERR_ARG, "tree_from_acceptance: null pointer");
  MEDUSA_REQUIRE(H >= 1 && K >= 1 && n_nodes >= 1 && n_nodes <= MEDUSA_MAX_TREE, MEDUSA_ERR_ARG,
                 "tree_from_acceptance: H=%d K=%d n_nodes=%d", H, K, n_nodes);
  double full = 0.0, level = 1.0;  // paths of the full K-ary tree of depth H
  for (int d = 0; d < H && full < n_nodes; ++d) {
    level *= K;
    full += level;
  }
  MEDUSA_REQUIRE(n_nodes - 1 <= full, MEDUSA_ERR_ARG, "tree_from_acceptance: %d nodes > the full tree", n_nodes);
  for (int d = 0; d < H; ++d) {
    double sum = 0.0;
    for (int r = 0; r < K; ++r) {
      const double a = acc[(size_t)d * K + r];
      MEDUSA_REQUIRE(a >= 0.0 && a <= 1.0, MEDUSA_ERR_ARG, "tree_from_acceptance: acc[%d][%d] = %g", d, r, a);
      sum += a;
    }
    MEDUSA_REQUIRE(sum <= 1.0 + 1e-9, MEDUSA_ERR_ARG, "tree_from_acceptance: depth %d rates sum to %g", d, sum);
  }
  // best-first: a path is never more probable than its parent and ties pop the
  // parent first, so paths come out in the global order
  std::priority_queue<Cand, std::vector<Cand>, After> heap;
  for (int r = 0; r < K; ++r) heap.push(Cand{1.0 * acc[r], {r}});
  double sum = 0.0;
  int off = 0;
  offsets[0] = 0;
  for (int i = 0; i < n_nodes - 1; ++i) {
    Cand c = heap.top();
    heap.pop();
    for (int32_t r : c.path) ranks[off++] = r;
    offsets[i + 1] = off;
    sum += c.p;
    const int d = (int)c.path.size();
    if (d < H)
      for (int r = 0; r < K; ++r) {
        Cand ch{c.p * acc[(size_t)d * K + r], c.path};
        ch.path.push_back(r);
        heap.push(std::move(ch));
      }
  }
  if (expected) *expected = sum;
  return MEDUSA_OK;
}

extern "C" int medusa_head_hits(int N, int H, int K, const int32_t* topk, const int32_t* tokens, int n_tokens,
                                int64_t* counts, int64_t* positions, hipStream_t stream) {
  MEDUSA_REQUIRE(N >= 0 && H >= 1 && K >= 1 && n_tokens >= 0, MEDUSA_ERR_ARG, "head_hits: bad sizes");
  MEDUSA_REQUIRE((int64_t)H * K <= HITS_MAX_BINS, MEDUSA_ERR_UNSUPPORTED, "head_hits: H*K = %d > %d", H * K,
                 HITS_MAX_BINS);
  if (N == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(topk && tokens && counts && positions, MEDUSA_ERR_ARG, "head_hits: null pointer");
  const int64_t pairs = (int64_t)N * H;
  int64_t blocks = (pairs + HITS_THREADS - 1) / HITS_THREADS;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(head_hits_kernel, dim3((unsigned)blocks), dim3(HITS_THREADS), 0, stream, N, H, K, topk, tokens,
                     n_tokens, (unsigned long long*)counts, (unsigned long long*)positions);
  return check_launch("head_hits");
}
