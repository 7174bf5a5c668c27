// Drives the library's host-side C++ (the static-tree builder and the tree
// calibration search) from a text description of the cases, for a build of
// those sources with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host code.  Input lines (stdin):
//   tree K n r0 r1 ... (n choices, each "len rank...")      -> tree buffers or status
//   accept H K n a_0 ... a_{H*K-1}                           -> chosen paths + expected length, or status
// Output: one line per input line, parsed by tests/test_host_sanitizers.py.
#include <stdio.h>
#include <stdlib.h>

#include <string>
#include <vector>

#include "medusa.h"

int main() {
  char kind[16];
  while (scanf("%15s", kind) == 1) {
    if (std::string(kind) == "tree") {
      int K, n;
      if (scanf("%d %d", &K, &n) != 2) return 2;
      std::vector<int32_t> ranks, offsets{0};
      for (int c = 0; c < n; ++c) {
        int len;
        if (scanf("%d", &len) != 1) return 2;
        for (int j = 0; j < len; ++j) {
          int r;
          if (scanf("%d", &r) != 1) return 2;
          ranks.push_back(r);
        }
        offsets.push_back((int32_t)ranks.size());
      }
      if (ranks.empty()) ranks.push_back(0);
      medusa_tree_host h;
      const int rc = medusa_tree_build_host(ranks.data(), offsets.data(), n, K, &h);
      if (rc) {
        printf("status %d\n", rc);
        continue;
      }
      printf("ok T %d D %d P %d K %d ti", h.T, h.D, h.P, h.K);
      for (int i = 0; i < h.T; ++i) printf(" %d", h.tree_indices[i]);
      printf(" parent");
      for (int i = 0; i < h.T; ++i) printf(" %d", h.parent[i]);
      printf(" anc");
      for (int i = 0; i < h.T; ++i) printf(" %llu", (unsigned long long)h.anc[i]);
      printf(" retrieve");
      for (int p = 0; p < h.P; ++p)
        for (int j = 0; j <= h.D; ++j) printf(" %d", h.retrieve[p * MEDUSA_MAX_TREE + j]);
      printf("\n");
    } else if (std::string(kind) == "accept") {
      int H, K, n;
      if (scanf("%d %d %d", &H, &K, &n) != 3) return 2;
      std::vector<double> acc((size_t)H * K);
      for (auto& a : acc)
        if (scanf("%lf", &a) != 1) return 2;
      std::vector<int32_t> ranks((size_t)(n > 1 ? n - 1 : 1) * H), offsets((size_t)(n > 0 ? n : 1));
      double expected = 0.0;
      const int rc = medusa_tree_from_acceptance(acc.data(), H, K, n, ranks.data(), offsets.data(), &expected);
      if (rc) {
        printf("status %d\n", rc);
        continue;
      }
      printf("ok %.17g", expected);
      for (int i = 0; i + 1 < n; ++i) {
        printf(" |");
        for (int k = offsets[i]; k < offsets[i + 1]; ++k) printf(" %d", ranks[k]);
      }
      printf("\n");
    } else {
      return 3;
    }
  }
  return 0;
}
