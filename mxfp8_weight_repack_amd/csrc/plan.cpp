// plan.cpp -- host planner: resolves the data tree, validates it, groups the
// update units and lays out the kernels' work tables.
//
// [SS-HSDP §3.2 "Data Tree"]: a child node is a view at an offset inside its
// parent; only the root owns storage and children reach it through their
// accumulated offset ("finalisation resolves child offsets", Appendix A).
// [SS-HSDP §3.3]: compatible parameters are grouped so their updates batch;
// [SS-HSDP §4.1]: the Newton-Schulz stage groups matrices with matching shapes
// and layouts into batched GEMMs.  [SS-HSDP Appendix A, Table 4]: planning
// rejects incompatible metadata, invalid geometry and storage overlap.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <tuple>
#include <new>
#include <utility>

#include "internal.h"

using namespace sshdp;

namespace {

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Interval {
  int64_t start, len;
  int32_t opt;    // SSHDP_OPT_* of the owning unit
  int32_t node;
};

// Row runs of a 2-D view: one interval if contiguous, else one per row.
void view_intervals(int64_t abs, int64_t rows, int64_t cols, int64_t rs, int32_t opt, int32_t node,
                    std::vector<Interval> &out) {
  if (rows == 1 || rs == cols) {
    out.push_back({abs, rows * cols, opt, node});
  } else {
    for (int64_t i = 0; i < rows; ++i) out.push_back({abs + i * rs, cols, opt, node});
  }
}

bool any_overlap(std::vector<Interval> v) {
  std::sort(v.begin(), v.end(), [](const Interval &a, const Interval &b) { return a.start < b.start; });
  for (size_t i = 1; i < v.size(); ++i)
    if (v[i].start < v[i - 1].start + v[i - 1].len) return true;
  return false;
}

int validate(const sshdp_node *nodes, int32_t n, int64_t root_numel, int layout, std::vector<int64_t> &abs,
             std::vector<int64_t> &ext) {
  abs.assign(n, 0);
  ext.assign(n, 0);
  for (int32_t i = 0; i < n; ++i) {
    const sshdp_node &nd = nodes[i];
    if (nd.parent < -1 || nd.parent >= i) return SSHDP_ERR_TREE;
    const int64_t rs = nd.rows > 1 ? nd.row_stride : nd.cols;
    if (nd.rows < 1 || nd.cols < 1 || nd.offset < 0 || rs < nd.cols) return SSHDP_ERR_SCHEMA;
    const int64_t base = nd.parent < 0 ? 0 : abs[nd.parent];
    const int64_t pext = nd.parent < 0 ? root_numel : ext[nd.parent];
    const int64_t e = (nd.rows - 1) * rs + nd.cols;
    const int64_t a = base + nd.offset;
    if (nd.offset + e > pext || a + e > root_numel) return SSHDP_ERR_BOUNDS;
    if (nd.is_unit && nd.optimizer != SSHDP_OPT_MUON && nd.optimizer != SSHDP_OPT_ADAMW)
      return SSHDP_ERR_SCHEMA;
    if (nd.is_unit && nd.optimizer == SSHDP_OPT_MUON) {
      if (nd.rows < 2 || nd.cols < 2) return SSHDP_ERR_SCHEMA;
      if (a % 4 || rs % 4 || nd.cols % 4) return SSHDP_ERR_SCHEMA;
      if (nd.rows > kNsMaxEdge || nd.cols > kNsMaxEdge) return SSHDP_ERR_SCHEMA;
    }
    if (nd.quantize != SSHDP_G_NONE && nd.quantize != SSHDP_G_MXFP8 && nd.quantize != SSHDP_G_BF16)
      return SSHDP_ERR_SCHEMA;
    if (nd.quantize == SSHDP_G_BF16) {
      if (rs != nd.cols || nd.cols % 8 || a % 8 || nd.cols > (1 << 30)) return SSHDP_ERR_SCHEMA;
    }
    if (nd.quantize == SSHDP_G_MXFP8) {
      if (rs != nd.cols || nd.cols % 32 || a % 32) return SSHDP_ERR_SCHEMA;
      if (layout == SSHDP_SCALE_TILE32X4 && (nd.rows % 32 || nd.cols % 128)) return SSHDP_ERR_SCHEMA;
      if (layout == SSHDP_SCALE_BLOCK32X32 && (nd.rows % 32 || a % 1024)) return SSHDP_ERR_SCHEMA;
      if (nd.cols > (1 << 30) || nd.rows > INT32_MAX) return SSHDP_ERR_SCHEMA;
    }
    abs[i] = a;
    ext[i] = e;
  }
  std::vector<Interval> units, quant;
  for (int32_t i = 0; i < n; ++i) {
    const sshdp_node &nd = nodes[i];
    const int64_t rs = nd.rows > 1 ? nd.row_stride : nd.cols;
    if (nd.is_unit) view_intervals(abs[i], nd.rows, nd.cols, rs, nd.optimizer, i, units);
  }
  if (any_overlap(units)) return SSHDP_ERR_OVERLAP;
  for (int32_t i = 0; i < n; ++i)
    if (nodes[i].quantize != SSHDP_G_NONE) quant.push_back({abs[i], nodes[i].rows * nodes[i].cols, 0, i});
  if (any_overlap(quant)) return SSHDP_ERR_OVERLAP;
  return SSHDP_OK;
}

float scale_factor(int mode, int64_t rows, int64_t cols) {
  if (mode == 1) return (float)std::sqrt(std::max(1.0, (double)rows / (double)cols));
  if (mode == 2) return (float)(0.2 * std::sqrt((double)std::max(rows, cols)));
  return 1.0f;
}


// Order one stage's tiles for the 8 XCDs of an MI355X (workgroup id i runs on
// XCD i % 8, each XCD with its own L2): tiles are cut into super-tiles per
// unit, super-tiles are dealt to XCDs, and each XCD's queue is laid out on the
// positions i = x (mod 8).  Workgroups that run together on one XCD then share
// their operand rows and columns through that L2.  Super-tiles are 4 x 4
// tiles, except for updates with K >= 4096, whose 8 x 4 super-tile is exactly
// the 32 workgroups an XCD runs at once (12 operand panels for 32 tiles); the
// former 8 x 8 measured 2.5% slower on the MoE bank and 2.2% on the d=8192
// block.  Tiles of equal K are ordered among themselves only (longer-K tiles
// stay first).
void xcd_order(std::vector<NsTile> &v, const std::vector<Group> &groups, bool gram, bool update) {
  constexpr int kXcd = 8;
  size_t s = 0;
  while (s < v.size()) {
    auto kof = [&](const NsTile &t) { return gram ? groups[t.group].c_pad : groups[t.group].r_pad; };
    size_t e = s;
    while (e < v.size() && kof(v[e]) == kof(v[s])) ++e;
    const int sm = update && kof(v[s]) >= 4096 ? 8 : 4, sn = 4;   // super-tile rows x columns (in tiles)
    // super-tiles in first-appearance order
    std::map<std::tuple<int, int, int, int>, size_t> idx;
    std::vector<std::vector<NsTile>> st;
    for (size_t i = s; i < e; ++i) {
      const auto key = std::make_tuple(v[i].group, v[i].b, v[i].tm / sm, v[i].tn / sn);
      auto it = idx.find(key);
      if (it == idx.end()) {
        idx[key] = st.size();
        st.push_back({v[i]});
      } else {
        st[it->second].push_back(v[i]);
      }
    }
    std::vector<std::vector<NsTile>> q(kXcd);
    for (auto &sup : st) {                           // deal to the least-loaded XCD
      size_t best = 0;
      for (size_t x = 1; x < q.size(); ++x)
        if (q[x].size() < q[best].size()) best = x;
      q[best].insert(q[best].end(), sup.begin(), sup.end());
    }
    std::vector<size_t> head(kXcd, 0);
    for (size_t pos = s; pos < e; ++pos) {
      size_t x = pos % kXcd;
      if (head[x] >= q[x].size()) {                  // this XCD's queue ran dry: take from the fullest
        size_t best = x;
        for (size_t y = 0; y < q.size(); ++y)
          if (q[y].size() - head[y] > q[best].size() - head[best]) best = y;
        x = best;
      }
      v[pos] = q[x][head[x]++];
    }
    s = e;
  }
}

void build_muon(sshdp_plan &p, const sshdp_node *nodes, int32_t n) {
  std::map<std::pair<int64_t, int64_t>, std::vector<int32_t>> by_shape;  // ordered: deterministic
  for (int32_t i = 0; i < n; ++i) {
    if (!nodes[i].is_unit || nodes[i].optimizer != SSHDP_OPT_MUON) continue;
    const int64_t r = std::min(nodes[i].rows, nodes[i].cols), c = std::max(nodes[i].rows, nodes[i].cols);
    by_shape[{r, c}].push_back(i);
  }
  p.node_group.assign(n, -1);
  size_t off = 0;
  const int64_t n_muon = [&] {
    int64_t k = 0;
    for (auto &kv : by_shape) k += (int64_t)kv.second.size();
    return k;
  }();
  p.ws_uscale = off;
  off = round_up(off + n_muon * sizeof(float), kAlign);
  // f0 tiles first (they size the partials buffer)
  for (auto &kv : by_shape) {
    Group g{};
    g.r = (int32_t)kv.first.first;
    g.c = (int32_t)kv.first.second;
    g.n = (int32_t)kv.second.size();
    {
      // Padding is to 128.  The largest 256-aligned leading block of each product runs in
      // 256 x 256 tiles where the group has enough of them to fill the machine (update: >= 128
      // tiles; Gram/poly: >= 192 triangle tiles, and r >= 4096 so the poly's contraction is
      // long enough to amortise a 256-tile's fill and two-sided store); the ragged strip
      // beyond it, or the whole product otherwise, in 128 x 128 tiles.  (MoE r = 1408: the
      // update in 256-tiles over 1280 rows plus a 128 strip, the Gram/poly in 128-tiles;
      // padding to 1536 instead costs 19% more flops.)
      g.r_pad = (int32_t)round_up(g.r, kNsSmall);
      g.c_pad = (int32_t)round_up(g.c, kNsSmall);
      const int64_t R2 = g.r_pad / kNsLarge, C2 = g.c_pad / kNsLarge;   // whole 256-tiles per edge
      const bool small = (p.opts.flags & SSHDP_PLAN_NS_TILES_SMALL) != 0;
      const bool large = (p.opts.flags & SSHDP_PLAN_NS_TILES_LARGE) != 0;
      const bool big = !small && (large || g.r >= 1024);
      const bool upd = big && R2 * C2 > 0 && (large || R2 * C2 * g.n >= 128);
      const bool gram = big && R2 > 0 && (large || (R2 * (R2 + 1) / 2 * g.n >= 192 && g.r >= 4096));
      g.u256r = upd ? (int32_t)(R2 * kNsLarge) : 0;
      g.u256c = upd ? (int32_t)(C2 * kNsLarge) : 0;
      g.g256 = gram ? (int32_t)(R2 * kNsLarge) : 0;
      // 128-tile Grams read X^T through transposing LDS reads, so the update stores X^T
      // only (and f0 only u^T): on those shapes the transposing read costs the Gram
      // 4-10% while the single-output epilogue saves ~8% of every update, more where
      // the update's K is short (MoE r = 1408).  256-tile Grams lose ~10% that way and
      // keep the NT form.
      // The K-major operand is all of X^T (c_pad x r_pad) behind one buffer resource, so
      // its byte offsets must stay below 2^31; larger units, and plans asking for it,
      // read X row-major.
      const bool km_fits = ((int64_t)g.c_pad - 1) * g.r_pad * 2 + kNsLarge * 2 <= (int64_t)0x7FFFFFFF;
      g.km = g.g256 == 0 && km_fits && !(p.opts.flags & SSHDP_PLAN_NS_GRAM_NT) ? 1 : 0;
      // One 128-row tile in r (per-head units, small matrices): B goes to memory as a pair of
      // bf16 matrices, its rounding and the remainder, and the update contracts over both
      // (K = 2 r_pad).  Rounding B to bf16 is the largest of the iteration's storage errors
      // (a 32 x 507 unit: 2.4e-2 from the float64 iteration with B in bf16, 1.2e-2 with the
      // pair); the doubled K costs these short-K, latency-bound updates little.
      g.split = g.r_pad == kNsSmall ? 1 : 0;
    }
    g.n = (int32_t)kv.second.size();
    g.unit_base = (int32_t)p.munits.size();
    const int gi = (int)p.groups.size();
    for (int32_t k = 0; k < g.n; ++k) {
      const int32_t ni = kv.second[k];
      const sshdp_node &nd = nodes[ni];
      MuonUnit u{};
      u.abs = p.node_abs[ni];
      u.row_stride = nd.rows > 1 ? nd.row_stride : nd.cols;
      u.rows = (int32_t)nd.rows;
      u.cols = (int32_t)nd.cols;
      u.tall = nd.rows > nd.cols ? 1 : 0;
      u.group = gi;
      u.idx = k;
      u.upd_scale = scale_factor(p.opts.muon_scale_mode, nd.rows, nd.cols);
      const int64_t Rp = u.tall ? g.c_pad : g.r_pad, Cp = u.tall ? g.r_pad : g.c_pad;
      u.Rp = (int32_t)Rp;
      u.Cp = (int32_t)Cp;
      u.tile_begin = (int32_t)p.f0tiles.size();
      for (int64_t tr = 0; tr < Rp / kF0Tile; ++tr)
        for (int64_t tc = 0; tc < Cp / kF0Tile; ++tc)
          p.f0tiles.push_back({(int32_t)p.munits.size(), (int32_t)tr, (int32_t)tc});
      u.tile_end = (int32_t)p.f0tiles.size();
      p.node_group[ni] = gi;
      p.munits.push_back(u);
      p.stats.muon_elems += nd.rows * nd.cols;
      p.stats.ns_flops += (double)p.opts.ns_steps *
                          (4.0 * (double)g.r * g.r * g.c + 2.0 * (double)g.r * g.r * g.r);
    }
    p.groups.push_back(g);
  }
  p.ws_partials = off;
  off = round_up(off + p.f0tiles.size() * sizeof(float), kAlign);
  for (Group &g : p.groups) {
    const size_t xs = (size_t)g.n * g.r_pad * g.c_pad * 2, as = (size_t)g.n * g.r_pad * g.r_pad * 2;
    g.off_x = off;   off = round_up(off + (g.km ? 0 : xs), kAlign);   // X is not stored for K-major Grams
    g.off_xt0 = off; off = round_up(off + xs, kAlign);
    g.off_xt1 = off; off = round_up(off + xs, kAlign);
    g.off_a = off;   off = round_up(off + as, kAlign);
    g.off_b = off;   off = round_up(off + (g.split ? 2 * as : as), kAlign);
    for (int32_t k = 0; k < g.n; ++k) {
      MuonUnit &u = p.munits[g.unit_base + k];
      const int64_t ux = (int64_t)g.off_x + (int64_t)k * g.r_pad * g.c_pad * 2;
      const int64_t ut = (int64_t)g.off_xt0 + (int64_t)k * g.r_pad * g.c_pad * 2;
      u.ws_orig = u.tall ? ut : ux;     // a tall unit's own layout is X^T
      u.ws_trans = u.tall ? ux : ut;
      if (g.km) (u.tall ? u.ws_trans : u.ws_orig) = -1;   // only X^T is stored
    }
  }
  p.ws_bytes = off;
  // per-group cost (executed MFMA flops per NS step), groups dealt to lanes largest first
  std::vector<double> cost(p.groups.size(), 0.0);
  for (size_t gi = 0; gi < p.groups.size(); ++gi) {
    const Group &g = p.groups[gi];
    const double L = kNsLarge, S = kNsSmall;
    const double n2 = g.g256 / kNsLarge, n1 = g.r_pad / kNsSmall, s1 = g.g256 / kNsSmall;
    const double tri = n2 * (n2 + 1) / 2 * L * L + ((n1 * (n1 + 1) - s1 * (s1 + 1)) / 2) * S * S;
    const double u2 = (double)(g.u256r / kNsLarge) * (g.u256c / kNsLarge) * L * L;
    const double u1 = ((double)g.r_pad * g.c_pad - (double)g.u256r * g.u256c);
    cost[gi] = g.n * (tri * 2.0 * (g.c_pad + g.r_pad) + (u2 + u1) * 2.0 * g.r_pad * (g.split ? 2 : 1));
    p.group_unit_flops.push_back(cost[gi] / g.n * p.opts.ns_steps);
  }
  std::vector<size_t> order(p.groups.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return cost[x] > cost[y]; });
  // The largest group takes the caller's stream (lane 0); the others are dealt,
  // largest first, to as few side streams as keep each side stream's load within
  // lane 0's: side work that finishes inside the critical path anyway, with
  // fewer side kernels contending for the CUs at once (d=2048 block: the O
  // projection and the 24 heads on one side stream, 2.44 ms per step against
  // 2.47 on two).  Once kMaxLanes are open, the least-loaded lane takes the rest.
  // When the largest group fills the GPU by itself, every group stays on lane 0.
  p.group_lane.assign(p.groups.size(), 0);
  p.n_lanes = 1;
  {
    std::vector<double> load(kMaxLanes, 0.0);
    if (!order.empty()) load[0] = cost[order[0]];
    // Side streams only pay off while the largest group's launches leave workgroup slots
    // idle (fewer than two rounds of the GPU's slots in some stage: e.g. the d=2048 block's
    // MLP Gram, 408 128-tiles in 512 slots).  When every stage of it fills the GPU at least
    // twice over, side kernels only take CUs from it: the d=8192 block runs 2% faster per
    // step with every group on the caller's stream (93.6 against 95.7 ms, same GPU), and the
    // d=2048 block 5% slower (2.43 against 2.31 ms).
    bool fills = !order.empty();
    if (fills) {
      const Group &g = p.groups[order[0]];
      const int64_t n2 = g.g256 / kNsLarge, n1 = g.r_pad / kNsSmall, s1 = g.g256 / kNsSmall;
      const int64_t tri256 = n2 * (n2 + 1) / 2 * g.n, tri128 = (n1 * (n1 + 1) - s1 * (s1 + 1)) / 2 * g.n;
      const int64_t up256 = (int64_t)(g.u256r / kNsLarge) * (g.u256c / kNsLarge) * g.n;
      const int64_t up128 = ((int64_t)g.r_pad * g.c_pad - (int64_t)g.u256r * g.u256c) / (kNsSmall * kNsSmall) * g.n;
      // rounds of one stage's launches: 256-tiles one per CU, 128-tiles two per CU
      auto rounds = [&](int64_t t256, int64_t t128) {
        return (double)t256 / kGpuCus + (double)t128 / (2.0 * kGpuCus);
      };
      fills = rounds(tri256, tri128) >= 2.0 && rounds(up256, up128) >= 2.0;
    }
    const bool one = (p.opts.flags & SSHDP_PLAN_NS_ONE_STREAM) != 0;
    // ... except groups that run in 128-tiles alone (r_pad == 128: per-head units), whose
    // short, latency-bound launches then run beside the big ones on one side stream (d=8192
    // block: 89.36 against 89.92 ms per step, same GPU, the update launch unchanged)
    if (fills && !one) {
      for (size_t k = 1; k < order.size(); ++k)
        if (p.groups[order[k]].r_pad == kNsSmall) {
          p.group_lane[order[k]] = 1;
          p.n_lanes = 2;
        }
    }
    for (size_t k = 1; k < order.size() && !one && !fills; ++k) {
      const double c = cost[order[k]];
      int best = -1;
      for (int l = 1; l < p.n_lanes; ++l)
        if (load[l] + c <= load[0] && (best < 0 || load[l] < load[best])) best = l;
      if (best < 0) {
        if (p.n_lanes < kMaxLanes) {
          best = p.n_lanes++;
        } else {
          best = 0;
          for (int l = 1; l < p.n_lanes; ++l)
            if (load[l] < load[best]) best = l;
        }
      }
      p.group_lane[order[k]] = best;
      load[best] += c;
    }
  }
  // f0 tiles and norm units regrouped by lane, so each lane runs its own f0 and norm
  // (the side lanes' then overlap lane 0's first Gram)
  {
    std::vector<F0Tile> tiles;
    tiles.reserve(p.f0tiles.size());
    p.norm_units.clear();
    for (int ln = 0; ln < p.n_lanes; ++ln) {
      p.f0_lane[ln] = (int32_t)tiles.size();
      p.norm_lane[ln] = (int32_t)p.norm_units.size();
      for (size_t gi = 0; gi < p.groups.size(); ++gi) {
        if (p.group_lane[gi] != ln) continue;
        for (int32_t k = 0; k < p.groups[gi].n; ++k) {
          const int32_t ui = p.groups[gi].unit_base + k;
          MuonUnit &u = p.munits[ui];
          const int32_t b = (int32_t)tiles.size();
          tiles.insert(tiles.end(), p.f0tiles.begin() + u.tile_begin, p.f0tiles.begin() + u.tile_end);
          u.tile_begin = b;
          u.tile_end = (int32_t)tiles.size();
          p.norm_units.push_back(ui);
        }
      }
    }
    for (int ln = p.n_lanes; ln <= kMaxLanes; ++ln) {
      p.f0_lane[ln] = (int32_t)tiles.size();
      p.norm_lane[ln] = (int32_t)p.norm_units.size();
    }
    p.f0tiles.swap(tiles);
  }
  // Stage outputs that the next stage reads back (X, X^T, A, B) are stored cacheable when the
  // NS working set of all groups, which run concurrently on the lanes, fits the last-level
  // cache; otherwise they would only evict operand lines and are stored nontemporal.
  int64_t ns_set = 0;
  for (const Group &g : p.groups)
    ns_set += (int64_t)g.n * g.r_pad * (g.c_pad + 2 * g.r_pad) * 2;
  p.ns_cached = ns_set <= kNsCacheBytes;
  // per-lane, per-stage tile tables: symmetric Gram/poly take tm <= tn; longest K first
  for (size_t gi = 0; gi < p.groups.size(); ++gi) {
    const Group &g = p.groups[gi];
    p.ns_groups.push_back({(int64_t)g.off_x, (int64_t)g.off_xt0, (int64_t)g.off_xt1, (int64_t)g.off_a,
                           (int64_t)g.off_b, g.r_pad, g.c_pad, g.unit_base, g.n, g.km, g.split});
    const int ln = p.group_lane[gi];
    const int n2 = g.g256 / kNsLarge, n1 = g.r_pad / kNsSmall, s1 = g.g256 / kNsSmall;
    const int ur2 = g.u256r / kNsLarge, uc2 = g.u256c / kNsLarge;
    const int ur1 = g.u256r / kNsSmall, uc1 = g.u256c / kNsSmall, nr1 = g.r_pad / kNsSmall, nc1 = g.c_pad / kNsSmall;
    for (int b = 0; b < g.n; ++b) {
      // Gram/poly (symmetric, tm <= tn, mirrored): 256-tiles on [0, g256)^2, 128-tiles on
      // the column strip [g256, r_pad) (their mirrors fill the row strip)
      for (int tm = 0; tm < n2; ++tm)
        for (int tn = tm; tn < n2; ++tn) {
          p.ns_tiles[ln][0][1].push_back({(int32_t)gi, b, tm, tn});
          p.ns_tiles[ln][1][1].push_back({(int32_t)gi, b, tm, tn});
        }
      for (int tn = s1; tn < n1; ++tn)
        for (int tm = 0; tm <= tn; ++tm) {
          p.ns_tiles[ln][0][0].push_back({(int32_t)gi, b, tm, tn});
          p.ns_tiles[ln][1][0].push_back({(int32_t)gi, b, tm, tn});
        }
      // update: 256-tiles on [0, u256r) x [0, u256c), 128-tiles on the rest.  The 256-tiles go
      // column by column, so their super-tiles are dealt to the XCDs column-major: the XCDs
      // working at one time share X^T column panels (each read once from HBM, the rest from
      // the last-level cache) and cycle through B, which fits that cache (d=8192 block: 87.96
      // against 89.5 ms per step with row-major super-tiles, the update launch 0.516 against
      // 0.501 of bf16 peak, same GPU; d=2048 block 2.234 against 2.247 ms).
      for (int tn = 0; tn < uc2; ++tn)
        for (int tm = 0; tm < ur2; ++tm) p.ns_tiles[ln][2][1].push_back({(int32_t)gi, b, tm, tn});
      for (int tm = 0; tm < nr1; ++tm)
        for (int tn = 0; tn < nc1; ++tn)
          if (tm >= ur1 || tn >= uc1) p.ns_tiles[ln][2][0].push_back({(int32_t)gi, b, tm, tn});
    }
  }
  // A symmetric product whose 256-tiles end in a short last round (at most half the CUs busy
  // in it) hands that round's worth of off-diagonal 256-tiles to the 128-tile launch that
  // follows on the same stream, four 128-tiles each, so no round runs mostly empty (d=8192
  // block: its poly 2048 + 256 instead of 2112 tiles, 11.3 against 11.6 ms per step, same
  // GPU).  Only where every 256-tile of the launch has the same contraction length (the poly
  // always; the Gram when its groups share c).
  for (int ln = 0; ln < p.n_lanes; ++ln)
    for (int st = 0; st < 2; ++st) {
      std::vector<NsTile> &v = p.ns_tiles[ln][st][1];
      const size_t n = v.size(), rem = n % kGpuCus;
      if (n <= (size_t)kGpuCus || rem == 0 || rem > (size_t)kGpuCus / 2) continue;
      bool same_k = true;
      for (const NsTile &t : v)
        same_k &= (st == 0 ? p.groups[t.group].c_pad : p.groups[t.group].r_pad) ==
                  (st == 0 ? p.groups[v[0].group].c_pad : p.groups[v[0].group].r_pad);
      if (!same_k) continue;
      std::vector<NsTile> keep, moved;
      for (size_t i = n; i-- > 0;) {
        if (moved.size() < rem && v[i].tm < v[i].tn) moved.push_back(v[i]);
        else keep.push_back(v[i]);
      }
      if (moved.size() < rem) continue;
      std::reverse(keep.begin(), keep.end());
      v.swap(keep);
      for (auto it = moved.rbegin(); it != moved.rend(); ++it)
        for (int i = 0; i < 2; ++i)
          for (int j = 0; j < 2; ++j)
            p.ns_tiles[ln][st][0].push_back({it->group, it->b, 2 * it->tm + i, 2 * it->tn + j});
    }
  for (int ln = 0; ln < p.n_lanes; ++ln)
    for (int st = 0; st < 3; ++st)
      for (int sz = 0; sz < 2; ++sz) {
        std::vector<NsTile> &v = p.ns_tiles[ln][st][sz];
        std::stable_sort(v.begin(), v.end(), [&](const NsTile &x, const NsTile &y) {
          const Group &gx = p.groups[x.group], &gy = p.groups[y.group];
          return (st == 0 ? gx.c_pad : gx.r_pad) > (st == 0 ? gy.c_pad : gy.r_pad);
        });
        xcd_order(v, p.groups, st == 0, st == 2);
        const double t = sz ? kNsLarge : kNsSmall;
        for (const NsTile &x : v) {
          const Group &gx = p.groups[x.group];
          p.stats.ns_tile_flops += t * t * 2.0 * (st == 0 ? gx.c_pad : st == 2 && gx.split ? 2 * gx.r_pad : gx.r_pad);
        }
      }
  p.stats.ns_tile_flops *= p.opts.ns_steps;
  p.stats.n_muon_units = (int32_t)p.munits.size();
  p.stats.n_groups = (int32_t)p.groups.size();
}

void build_elementwise(sshdp_plan &p, const sshdp_node *nodes, int32_t n) {
  std::vector<Interval> units;
  for (int32_t i = 0; i < n; ++i) {
    const sshdp_node &nd = nodes[i];
    if (!nd.is_unit) continue;
    view_intervals(p.node_abs[i], nd.rows, nd.cols, nd.rows > 1 ? nd.row_stride : nd.cols, nd.optimizer, i,
                   units);
    if (nd.optimizer == SSHDP_OPT_ADAMW) {
      p.stats.n_adamw_units++;
      p.stats.adamw_elems += nd.rows * nd.cols;
    }
  }
  std::sort(units.begin(), units.end(), [](const Interval &a, const Interval &b) { return a.start < b.start; });
  std::vector<char> fused_node(n, 0);  // AdamW unit handled inside a fused region
  std::vector<QChunk> fused, plain;
  for (int32_t i = 0; i < n; ++i) {
    const sshdp_node &nd = nodes[i];
    if (nd.quantize == SSHDP_G_BF16) {
      const int64_t a = p.node_abs[i], len = nd.rows * nd.cols;
      for (int64_t pos = a; pos < a + len; pos += kChunk)
        p.cchunks.push_back({pos, (int32_t)std::min<int64_t>(kChunk, a + len - pos), 0});
      p.stats.cast_elems += len;
      p.stats.n_cast_regions++;
      continue;
    }
    if (nd.quantize != SSHDP_G_MXFP8) continue;
    const int32_t ri = (int32_t)p.qregions.size();
    const int64_t a = p.node_abs[i], len = nd.rows * nd.cols;
    p.qregions.push_back({a, nd.rows, (int32_t)nd.cols, 0});
    p.stats.quant_elems += len;
    if (p.opts.scale_layout == SSHDP_SCALE_BLOCK32X32) {
      // 32-row strips cut into tiles of up to 4 blocks; AdamW is not fused here
      const int64_t kb = nd.cols / 32;
      for (int64_t br = 0; br < nd.rows / 32; ++br)
        for (int64_t b0 = 0; b0 < kb; b0 += 4)
          p.q32tiles.push_back({a + br * 32 * nd.cols + b0 * 32, a / 1024 + br * kb + b0, (int32_t)nd.cols,
                                (int32_t)std::min<int64_t>(4, kb - b0)});
      continue;
    }
    // unit intervals intersecting the region
    auto it = std::lower_bound(units.begin(), units.end(), a,
                               [](const Interval &u, int64_t x) { return u.start + u.len <= x; });
    std::vector<Interval> inside;
    bool eligible = true;
    for (; it != units.end() && it->start < a + len; ++it) {
      if (it->start + it->len <= a) continue;
      inside.push_back(*it);
      if (it->opt != SSHDP_OPT_ADAMW) eligible = false;
      if (it->start < a || it->start + it->len > a + len) eligible = false;
    }
    // a region holding no unit has no AdamW to fuse: plain G chunks
    if (inside.empty()) eligible = false;
    // every AdamW unit touching the region must lie entirely inside it
    if (eligible) {
      for (const Interval &iv : inside) {
        const sshdp_node &un = nodes[iv.node];
        const int64_t rs = un.rows > 1 ? un.row_stride : un.cols;
        const int64_t ua = p.node_abs[iv.node], ue = ua + (un.rows - 1) * rs + un.cols;
        if (ua < a || ue > a + len) eligible = false;
      }
      for (size_t k = 1; k < inside.size() && eligible; ++k)   // no two runs share a block
        if ((inside[k].start / 32) <= ((inside[k - 1].start + inside[k - 1].len - 1) / 32)) eligible = false;
    }
    std::vector<QChunk> &dst = eligible ? fused : plain;
    size_t next = 0;
    int64_t pos = a;
    while (pos < a + len) {
      int64_t end = std::min(a + len, pos + (int64_t)kChunk);
      if (eligible) {
        // a new chunk starts at the block of every run start, so a chunk holds at most one run
        while (next < inside.size() && inside[next].start / 32 * 32 <= pos) ++next;
        if (next < inside.size()) {
          const int64_t rb = inside[next].start / 32 * 32;
          if (rb > pos && rb < end) end = rb;
        }
      }
      QChunk q{};
      q.base = pos;
      q.n = (int32_t)(end - pos);
      q.region = ri;
      q.row0 = (int32_t)((pos - a) / nd.cols);
      q.col0 = (int32_t)((pos - a) % nd.cols);
      q.lo = q.hi = pos;
      if (eligible) {
        for (const Interval &iv : inside) {
          const int64_t lo = std::max(iv.start, pos), hi = std::min(iv.start + iv.len, end);
          if (lo < hi) { q.lo = lo; q.hi = hi; break; }
        }
      }
      dst.push_back(q);
      pos = end;
    }
    if (eligible) {
      for (const Interval &iv : inside) fused_node[iv.node] = 1;
      p.stats.fused_quant_elems += len;
    }
  }
  p.n_qchunks_fused = (int64_t)fused.size();
  p.qchunks = fused;
  p.qchunks.insert(p.qchunks.end(), plain.begin(), plain.end());
  p.stats.n_quant_regions = (int32_t)p.qregions.size();
  for (const Interval &iv : units) {
    if (iv.opt != SSHDP_OPT_ADAMW) continue;
    for (int64_t s = iv.start; s < iv.start + iv.len; s += kChunk) {
      ASeg sg{s, (int32_t)std::min<int64_t>(kChunk, iv.start + iv.len - s), 0};
      p.aseg_all.push_back(sg);
      if (!fused_node[iv.node]) p.aseg_unfused.push_back(sg);
    }
  }
}

template <class T>
size_t table_bytes(const std::vector<T> &v) { return round_up((int64_t)(v.size() * sizeof(T)), 256); }

int upload(sshdp_plan &p) {
  const size_t total = table_bytes(p.munits) + table_bytes(p.f0tiles) + table_bytes(p.aseg_all) +
                       table_bytes(p.aseg_unfused) + table_bytes(p.qregions) + table_bytes(p.qchunks) +
                       table_bytes(p.q32tiles) + table_bytes(p.cchunks) + table_bytes(p.ns_groups) +
                       table_bytes(p.norm_units) + 256;
  size_t tiles_total = 0;
  for (auto &ln : p.ns_tiles)
    for (auto &st : ln)
      for (auto &v : st) tiles_total += table_bytes(v);
  if (hipGetDevice(&p.device) != hipSuccess) return SSHDP_ERR_HIP;
  const size_t all = total + tiles_total;
  if (hipMalloc(&p.dblock, all) != hipSuccess) { p.dblock = nullptr; return SSHDP_ERR_HIP; }
  std::vector<char> host(all, 0);
  size_t off = 0;
  auto put = [&](auto &vec, auto *&dptr) {
    using T = typename std::remove_reference<decltype(vec)>::type::value_type;
    if (!vec.empty()) std::memcpy(host.data() + off, vec.data(), vec.size() * sizeof(T));
    dptr = reinterpret_cast<T *>(static_cast<char *>(p.dblock) + off);
    off += table_bytes(vec);
  };
  put(p.munits, p.d.munits);
  put(p.f0tiles, p.d.f0tiles);
  put(p.aseg_all, p.d.aseg_all);
  put(p.aseg_unfused, p.d.aseg_unfused);
  put(p.qregions, p.d.qregions);
  put(p.qchunks, p.d.qchunks);
  put(p.q32tiles, p.d.q32tiles);
  put(p.cchunks, p.d.cchunks);
  put(p.ns_groups, p.d.ns_groups);
  put(p.norm_units, p.d.norm_units);
  for (int ln = 0; ln < kMaxLanes; ++ln)
    for (int st = 0; st < 3; ++st)
      for (int sz = 0; sz < 2; ++sz) put(p.ns_tiles[ln][st][sz], p.d.ns_tiles[ln][st][sz]);
  if (hipMemcpy(p.dblock, host.data(), all, hipMemcpyHostToDevice) != hipSuccess) return SSHDP_ERR_HIP;
  // side streams (default priority, non-blocking) and the events that fork/join them
  if (p.n_lanes > 1) {
    if (hipEventCreateWithFlags(&p.ev_fork, hipEventDisableTiming) != hipSuccess) return SSHDP_ERR_HIP;
    for (int ln = 1; ln < p.n_lanes; ++ln) {
      if (hipStreamCreateWithFlags(&p.lane_stream[ln], hipStreamNonBlocking) != hipSuccess) return SSHDP_ERR_HIP;
      if (hipEventCreateWithFlags(&p.ev_join[ln], hipEventDisableTiming) != hipSuccess) return SSHDP_ERR_HIP;
    }
  }
  return SSHDP_OK;
}

}  // namespace

extern "C" {

int sshdp_abi_version(void) { return SSHDP_ABI_VERSION; }

const char *sshdp_status_string(int code) {
  switch (code) {
    case SSHDP_OK: return "ok";
    case SSHDP_ERR_ARG: return "invalid argument";
    case SSHDP_ERR_TREE: return "data tree: parent is not an earlier node";
    case SSHDP_ERR_BOUNDS: return "view leaves its parent or the root";
    case SSHDP_ERR_OVERLAP: return "units or quantised regions share storage";
    case SSHDP_ERR_SCHEMA: return "geometry or metadata the kernels cannot take";
    case SSHDP_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case SSHDP_ERR_WORKSPACE: return "workspace missing or too small";
    case SSHDP_ERR_HIP: return "HIP runtime error";
    case SSHDP_ERR_STATE: return "plan is host-only";
    case SSHDP_ERR_SCRATCH: return "plan needs more workspace than the built-in scratch holds";
    default: return "unknown status";
  }
}

int sshdp_default_opts(sshdp_plan_opts *o) {
  if (!o) return SSHDP_ERR_ARG;
  o->ns_steps = 5;
  o->ns_a = 3.4445f;
  o->ns_b = -4.7750f;
  o->ns_c = 2.0315f;
  o->ns_eps = 1e-7f;
  o->scale_layout = SSHDP_SCALE_ROWMAJOR;
  o->nesterov = 0;
  o->muon_scale_mode = 0;
  o->flags = 0;
  return SSHDP_OK;
}

int sshdp_plan_views(const sshdp_node *nodes, int32_t n_nodes, int64_t root_numel, const sshdp_plan_opts *opts,
                     sshdp_plan **out_plan) {
  if (!out_plan) return SSHDP_ERR_ARG;
  *out_plan = nullptr;
  if (!nodes || n_nodes <= 0 || root_numel <= 0) return SSHDP_ERR_ARG;
  sshdp_plan_opts o;
  if (opts) o = *opts; else sshdp_default_opts(&o);
  if (o.ns_steps < 1 || o.ns_steps > 64 || (o.scale_layout != SSHDP_SCALE_ROWMAJOR &&
      o.scale_layout != SSHDP_SCALE_TILE32X4 && o.scale_layout != SSHDP_SCALE_BLOCK32X32) ||
      o.muon_scale_mode < 0 || o.muon_scale_mode > 2 ||
      !(o.ns_eps >= 0.0f) || (o.flags & ~31u) ||
      ((o.flags & SSHDP_PLAN_NS_TILES_SMALL) && (o.flags & SSHDP_PLAN_NS_TILES_LARGE)))
    return SSHDP_ERR_ARG;
  std::vector<int64_t> abs, ext;
  int st = validate(nodes, n_nodes, root_numel, o.scale_layout, abs, ext);
  if (st != SSHDP_OK) return st;
  sshdp_plan *p = new (std::nothrow) sshdp_plan();
  if (!p) return SSHDP_ERR_ARG;
  p->root_numel = root_numel;
  p->opts = o;
  p->node_abs = abs;
  p->stats.root_numel = root_numel;
  p->stats.scale_bytes = o.scale_layout == SSHDP_SCALE_BLOCK32X32 ? (root_numel + 1023) / 1024 : (root_numel + 31) / 32;
  p->stats.n_nodes = n_nodes;
  for (int32_t i = 0; i < n_nodes; ++i) p->stats.n_units += nodes[i].is_unit ? 1 : 0;
  build_muon(*p, nodes, n_nodes);
  build_elementwise(*p, nodes, n_nodes);
  p->stats.workspace_bytes = (int64_t)p->ws_bytes;
  p->host_only = (o.flags & SSHDP_PLAN_HOST_ONLY) != 0;
  if (!p->host_only) {
    st = upload(*p);
    if (st != SSHDP_OK) {
      sshdp_plan_destroy(p);
      return st;
    }
  }
  *out_plan = p;
  return SSHDP_OK;
}

int sshdp_plan_info(const sshdp_plan *p, sshdp_plan_stats *s) {
  if (!p || !s) return SSHDP_ERR_ARG;
  *s = p->stats;
  return SSHDP_OK;
}

int sshdp_plan_group(const sshdp_plan *p, int32_t g, sshdp_group_info *info) {
  if (!p || !info || g < 0 || g >= (int32_t)p->groups.size()) return SSHDP_ERR_ARG;
  const Group &G = p->groups[g];
  info->r = G.r; info->c = G.c; info->r_pad = G.r_pad; info->c_pad = G.c_pad;
  info->n_units = G.n; info->tile = G.u256r ? kNsLarge : kNsSmall; info->tile_gram = G.g256 ? kNsLarge : kNsSmall;
  info->gram256 = G.g256; info->upd256_rows = G.u256r; info->upd256_cols = G.u256c;
  info->gram_kmajor = G.km;
  info->split_b = G.split;
  info->lane = p->group_lane[g];
  return SSHDP_OK;
}

int sshdp_plan_node(const sshdp_plan *p, int32_t node, int64_t *abs_offset, int32_t *group) {
  if (!p || node < 0 || node >= (int32_t)p->node_abs.size()) return SSHDP_ERR_ARG;
  if (abs_offset) *abs_offset = p->node_abs[node];
  if (group) *group = p->node_group[node];
  return SSHDP_OK;
}

void sshdp_plan_destroy(sshdp_plan *p) {
  if (!p) return;
  if (p->dblock) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (p->device >= 0 && cur != p->device) (void)hipSetDevice(p->device);
    (void)hipFree(p->dblock);
    if (cur >= 0 && cur != p->device) (void)hipSetDevice(cur);
  }
  for (int ln = 1; ln < kMaxLanes; ++ln) {
    if (p->lane_stream[ln]) (void)hipStreamDestroy(p->lane_stream[ln]);
    if (p->ev_join[ln]) (void)hipEventDestroy(p->ev_join[ln]);
  }
  if (p->ev_fork) (void)hipEventDestroy(p->ev_fork);
  for (auto &e : p->prof_pending) { (void)hipEventDestroy(e.second.first); (void)hipEventDestroy(e.second.second); }
  for (hipEvent_t e : p->prof_pool) (void)hipEventDestroy(e);
  delete p;
}

}  // extern "C"
