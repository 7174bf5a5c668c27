// Error reporting and the static-tree builder (host side).
//
// The tree buffers follow generate_medusa_buffers() on the page "大模型推理
// memory bandwidth bound (5) - Medusa", section 二.2: nodes sorted by depth then
// ranks, tree_indices = 1 + K*(depth-1) + last rank, position ids = depth, the
// ancestor-or-self mask, and one retrieve row per leaf (decreasing leaf index,
// -1 padded).
#include <stdarg.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <vector>

#include "common.h"
#include "tree_dev.h"

namespace medusa {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MEDUSA_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return MEDUSA_OK;
}

}  // namespace medusa

using namespace medusa;

extern "C" const char* medusa_last_error(void) { return g_err; }
extern "C" int medusa_version(void) { return 1; }

extern "C" int medusa_tree_build_host(const int32_t* ranks, const int32_t* offsets, int32_t n_choices, int32_t K,
                                      medusa_tree_host* out) {
  MEDUSA_REQUIRE(out != nullptr, MEDUSA_ERR_ARG, "tree_create: out is null");
  MEDUSA_REQUIRE(n_choices >= 0, MEDUSA_ERR_ARG, "tree_create: n_choices < 0");
  MEDUSA_REQUIRE(n_choices == 0 || (ranks && offsets), MEDUSA_ERR_ARG, "tree_create: null ranks/offsets");
  MEDUSA_REQUIRE(n_choices + 1 <= MEDUSA_MAX_TREE, MEDUSA_ERR_UNSUPPORTED,
                 "tree_create: %d nodes exceed the %d-node limit", n_choices + 1, MEDUSA_MAX_TREE);
  std::vector<std::vector<int>> ch(n_choices);
  int maxrank = -1;
  for (int c = 0; c < n_choices; ++c) {
    int a = offsets[c], b = offsets[c + 1];
    MEDUSA_REQUIRE(b > a, MEDUSA_ERR_ARG, "tree_create: choice %d is empty", c);
    MEDUSA_REQUIRE(b - a < MEDUSA_MAX_TREE, MEDUSA_ERR_UNSUPPORTED, "tree_create: choice %d too deep", c);
    for (int k = a; k < b; ++k) {
      MEDUSA_REQUIRE(ranks[k] >= 0, MEDUSA_ERR_ARG, "tree_create: negative rank in choice %d", c);
      ch[c].push_back(ranks[k]);
      maxrank = std::max(maxrank, (int)ranks[k]);
    }
  }
  if (K <= 0) K = maxrank + 1 > 0 ? maxrank + 1 : 1;
  MEDUSA_REQUIRE(maxrank < K, MEDUSA_ERR_ARG, "tree_create: rank %d >= K=%d", maxrank, K);
  // sort by (depth, lexicographic ranks)
  std::sort(ch.begin(), ch.end(), [](const std::vector<int>& x, const std::vector<int>& y) {
    if (x.size() != y.size()) return x.size() < y.size();
    return x < y;
  });
  std::map<std::vector<int>, int> node_of;
  node_of[std::vector<int>()] = 0;
  for (int c = 0; c < n_choices; ++c) {
    MEDUSA_REQUIRE(node_of.find(ch[c]) == node_of.end(), MEDUSA_ERR_ARG, "tree_create: duplicate choice");
    node_of[ch[c]] = c + 1;
  }
  medusa_tree_host& h = *out;
  memset(&h, 0, sizeof(h));
  const int T = n_choices + 1;
  h.T = T;
  h.K = K;
  h.depth[0] = 0;
  h.parent[0] = -1;
  h.tree_indices[0] = 0;
  int D = 0;
  for (int c = 0; c < n_choices; ++c) {
    const std::vector<int>& p = ch[c];
    std::vector<int> par(p.begin(), p.end() - 1);
    auto it = node_of.find(par);
    MEDUSA_REQUIRE(it != node_of.end(), MEDUSA_ERR_ARG, "tree_create: a choice has no parent in the tree");
    const int i = c + 1;
    h.depth[i] = (int)p.size();
    h.parent[i] = it->second;
    h.tree_indices[i] = 1 + K * ((int)p.size() - 1) + p.back();
    D = std::max(D, (int)p.size());
  }
  h.D = D;
  h.H = D;
  // ancestor-or-self bitsets by walking parents
  for (int i = 0; i < T; ++i) {
    uint64_t m = 0;
    for (int j = i; j >= 0; j = h.parent[j]) m |= (uint64_t)1 << j;
    h.anc[i] = m;
  }
  // leaves in decreasing index
  std::vector<bool> is_parent(T, false);
  for (int i = 1; i < T; ++i) is_parent[h.parent[i]] = true;
  int P = 0;
  for (int i = 0; i < MEDUSA_MAX_TREE * MEDUSA_MAX_TREE; ++i) h.retrieve[i] = -1;
  for (int leaf = T - 1; leaf >= 0; --leaf) {
    if (is_parent[leaf]) continue;
    int len = h.depth[leaf] + 1;
    for (int j = leaf, k = len - 1; j >= 0; j = h.parent[j], --k) h.retrieve[P * MEDUSA_MAX_TREE + k] = j;
    h.path_len[P] = len;
    ++P;
  }
  h.P = P;

  return MEDUSA_OK;
}

extern "C" int medusa_tree_create(const int32_t* ranks, const int32_t* offsets, int32_t n_choices, int32_t K,
                                  medusa_tree** out) {
  MEDUSA_REQUIRE(out != nullptr, MEDUSA_ERR_ARG, "tree_create: out is null");
  *out = nullptr;
  medusa_tree_host h;
  int rc = medusa_tree_build_host(ranks, offsets, n_choices, K, &h);
  if (rc) return rc;
  medusa_tree* t = new medusa_tree;
  t->host = h;
  t->dev = nullptr;
  hipError_t e = hipMalloc((void**)&t->dev, sizeof(medusa_tree_host));
  if (e != hipSuccess) {
    delete t;
    return fail(MEDUSA_ERR_HIP, "tree_create: hipMalloc: %s", hipGetErrorString(e));
  }
  e = hipMemcpy(t->dev, &t->host, sizeof(medusa_tree_host), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(t->dev);
    delete t;
    return fail(MEDUSA_ERR_HIP, "tree_create: hipMemcpy: %s", hipGetErrorString(e));
  }
  *out = t;
  return MEDUSA_OK;
}

extern "C" int medusa_tree_info(const medusa_tree* t, medusa_tree_host* out) {
  MEDUSA_REQUIRE(t && out, MEDUSA_ERR_ARG, "tree_info: null argument");
  *out = t->host;
  return MEDUSA_OK;
}

extern "C" const uint64_t* medusa_tree_anc_device(const medusa_tree* t) {
  return t ? t->dev->anc : nullptr;
}

extern "C" int medusa_tree_destroy(medusa_tree* t) {
  if (!t) return MEDUSA_OK;
  hipError_t e = hipFree(t->dev);
  delete t;
  if (e != hipSuccess) return fail(MEDUSA_ERR_HIP, "tree_destroy: hipFree: %s", hipGetErrorString(e));
  return MEDUSA_OK;
}
