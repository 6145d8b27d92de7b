// Host-only driver of the planner for the sanitizer test: reads data trees from a
// binary file, plans each with SSHDP_PLAN_HOST_ONLY (no device), queries the plan
// and destroys it.  Built from plan.cpp with g++ -fsanitize=address,undefined by
// tests/test_planner_sanitized.py; prints one line per tree for comparison with
// the library's own host-only plans.
//
// File: repeated { int32 n_nodes; int64 root_numel; int32 layout; uint32 flags;
//                  sshdp_node nodes[n_nodes]; }
#include <cstdio>
#include <cstdint>
#include <vector>

#include "sshdp.h"

int main(int argc, char **argv) {
  if (argc != 2) return 2;
  FILE *f = std::fopen(argv[1], "rb");
  if (!f) return 2;
  for (int tree = 0;; ++tree) {
    int32_t n = 0;
    int64_t root = 0;
    int32_t layout = 0;
    uint32_t flags = 0;
    if (std::fread(&n, sizeof n, 1, f) != 1) break;
    if (std::fread(&root, sizeof root, 1, f) != 1 || std::fread(&layout, sizeof layout, 1, f) != 1 ||
        std::fread(&flags, sizeof flags, 1, f) != 1)
      return 3;
    std::vector<sshdp_node> nodes(n > 0 ? n : 0);
    if (n > 0 && std::fread(nodes.data(), sizeof(sshdp_node), n, f) != (size_t)n) return 3;
    sshdp_plan_opts o;
    sshdp_default_opts(&o);
    o.scale_layout = layout;
    o.flags = flags | SSHDP_PLAN_HOST_ONLY;
    sshdp_plan *p = nullptr;
    const int st = sshdp_plan_views(nodes.data(), n, root, &o, &p);
    if (st != SSHDP_OK) {
      std::printf("%d status %d\n", tree, st);
      if (p) return 4;                                  // errors leave the plan NULL
      continue;
    }
    sshdp_plan_stats s{};
    if (sshdp_plan_info(p, &s) != SSHDP_OK) return 5;
    std::printf("%d ok ws %lld scale %lld groups %d tileflops %.17g", tree, (long long)s.workspace_bytes,
                (long long)s.scale_bytes, s.n_groups, s.ns_tile_flops);
    for (int g = 0; g < s.n_groups; ++g) {
      sshdp_group_info gi{};
      if (sshdp_plan_group(p, g, &gi) != SSHDP_OK) return 6;
      std::printf(" [%d %d %d %d %d %d %d %d %d]", gi.r, gi.c, gi.r_pad, gi.c_pad, gi.n_units, gi.gram256,
                  gi.upd256_rows, gi.upd256_cols, gi.gram_kmajor);
    }
    for (int i = 0; i < n; ++i) {
      int64_t a = -1;
      int32_t g = -2;
      if (sshdp_plan_node(p, i, &a, &g) != SSHDP_OK) return 7;
    }
    std::printf("\n");
    sshdp_plan_destroy(p);
  }
  std::fclose(f);
  return 0;
}
