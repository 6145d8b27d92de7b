// Host-only check of the launching entry points' stream ordering on error paths.
// Built by tests/test_api_error_paths.py with g++ from plan.cpp and api.hip (which
// launches nothing itself) against a stand-in of the few HIP runtime calls they make
// and of the kernel launchers: streams and events are plain host objects, every
// event record / stream wait is logged, and the n-th launcher call fails.  For
// every n, a step must return SSHDP_ERR_HIP (or OK once n exceeds the launches of a
// whole step) and leave every side stream it forked joined back into the caller's
// stream: the side stream's last logged operation is a record of its join event,
// and the caller's stream waits on that event afterwards.
//
// Input: one tree in the format of host_planner_check.cpp (first record only).
//
// With a second argument "tiles", the program instead checks the Newton-Schulz
// tile tables of every record in the file, for each tile policy: per unit, the
// Gram and poly tiles cover each 128 x 128 cell of the upper triangle of
// r_pad x r_pad exactly once (256-tiles count for their 2 x 2 cells, a diagonal
// one for its 3 upper cells), the update tiles cover every cell of r_pad x c_pad
// exactly once, and every tile of a group sits in its group's lane.
#include <cstdio>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "internal.h"

struct ihipStream_t { int id; };
struct ihipEvent_t { int id; };

namespace {
struct Op {
  char kind;   // 'R' record(event, stream), 'W' wait(stream, event), 'L' launch(stream)
  int stream, event;
};
std::vector<Op> g_log;
int g_launch = 0, g_fail_at = -1, g_next_id = 1;

int sid(hipStream_t s) { return s ? s->id : 0; }   // 0: the null stream

hipError_t launched(hipStream_t s) {
  ++g_launch;
  g_log.push_back({'L', sid(s), 0});
  return g_launch == g_fail_at ? hipErrorLaunchFailure : hipSuccess;
}
}  // namespace

extern "C" {
hipError_t hipMalloc(void **p, size_t n) { *p = std::malloc(n ? n : 1); return *p ? hipSuccess : hipErrorOutOfMemory; }
hipError_t hipFree(void *p) { std::free(p); return hipSuccess; }
hipError_t hipMemcpy(void *d, const void *s, size_t n, hipMemcpyKind) { std::memcpy(d, s, n); return hipSuccess; }
hipError_t hipMemcpyAsync(void *d, const void *s, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(d, s, n);
  return hipSuccess;
}
hipError_t hipGetDevice(int *d) { *d = 0; return hipSuccess; }
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipStreamCreateWithFlags(hipStream_t *s, unsigned) { *s = new ihipStream_t{g_next_id++}; return hipSuccess; }
hipError_t hipStreamDestroy(hipStream_t s) { delete s; return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipEventCreate(hipEvent_t *e) { *e = new ihipEvent_t{g_next_id++}; return hipSuccess; }
hipError_t hipEventCreateWithFlags(hipEvent_t *e, unsigned) { *e = new ihipEvent_t{g_next_id++}; return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t e) { delete e; return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float *ms, hipEvent_t, hipEvent_t) { *ms = 0.f; return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s) { g_log.push_back({'R', sid(s), e->id}); return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned) {
  g_log.push_back({'W', sid(s), e->id});
  return hipSuccess;
}
}  // extern "C"

namespace sshdp {
hipError_t launch_f0(const sshdp_plan &, int, const float *, float *, float, int, char *, hipStream_t s) {
  return launched(s);
}
hipError_t launch_norm(const sshdp_plan &, int, char *, float, hipStream_t s) { return launched(s); }
hipError_t launch_ns_stage(const sshdp_plan &, int, int, int, char *, float *, float, float, hipStream_t s, int) {
  return launched(s);
}
hipError_t launch_gemm_raw(const void *, const void *, const void *, void *, void *, int, int, int, int, float, float,
                           int, hipStream_t s) {
  return launched(s);
}
hipError_t launch_adamw(const ASeg *, int64_t, const sshdp_buffers &, const sshdp_adamw_hp &, int64_t, hipStream_t s) {
  return launched(s);
}
hipError_t launch_quant(const sshdp_plan &, int64_t, int64_t, bool, const sshdp_buffers &, const sshdp_adamw_hp *,
                        int64_t, hipStream_t s) {
  return launched(s);
}
hipError_t launch_quant32(const sshdp_plan &, const float *, uint8_t *, uint8_t *, hipStream_t s) { return launched(s); }
hipError_t launch_cast_bf16(const sshdp_plan &, const float *, uint16_t *, hipStream_t s) { return launched(s); }
hipError_t launch_rs_reduce(const void *const *, int, int, void *, int, int64_t, uint64_t, uint64_t, int64_t,
                            hipStream_t s) {
  return launched(s);
}
hipError_t launch_rs_accumulate(const void *const *, int, int, float *, int64_t, int, hipStream_t s) {
  return launched(s);
}
}  // namespace sshdp

namespace {
// Every side stream that took part in the call ends with a record of an event the
// caller's stream waits on later.
bool joined(int caller, int *bad_stream) {
  std::vector<int> side;
  for (const Op &o : g_log)
    if (o.stream != caller) {
      bool seen = false;
      for (int x : side) seen |= x == o.stream;
      if (!seen) side.push_back(o.stream);
    }
  for (int l : side) {
    int last = -1;
    for (int i = 0; i < (int)g_log.size(); ++i)
      if (g_log[i].stream == l) last = i;
    bool ok = g_log[last].kind == 'R';
    if (ok) {
      ok = false;
      for (int i = last + 1; i < (int)g_log.size(); ++i)
        ok |= g_log[i].kind == 'W' && g_log[i].stream == caller && g_log[i].event == g_log[last].event;
    }
    if (!ok) {
      *bad_stream = l;
      return false;
    }
  }
  return true;
}

// 0 if every table covers its unit's cells exactly once; else prints the first
// problem and returns nonzero.
int check_tiles(const sshdp_plan &p, const char *what) {
  for (size_t gi = 0; gi < p.groups.size(); ++gi) {
    const sshdp::Group &g = p.groups[gi];
    const int R = g.r_pad / sshdp::kNsSmall, C = g.c_pad / sshdp::kNsSmall;
    for (int st = 0; st < 3; ++st) {
      const int W = st == 2 ? C : R;
      std::vector<int> cnt((size_t)g.n * R * W, 0);
      for (int ln = 0; ln < sshdp::kMaxLanes; ++ln)
        for (int sz = 0; sz < 2; ++sz)
          for (const sshdp::NsTile &t : p.ns_tiles[ln][st][sz]) {
            if (t.group != (int)gi) continue;
            if (ln != p.group_lane[gi] || t.b < 0 || t.b >= g.n) {
              std::printf("%s group %zu stage %d: tile (b %d) on lane %d, group lane %d\n", what, gi, st, t.b, ln,
                          p.group_lane[gi]);
              return 7;
            }
            const int k = sz ? 2 : 1;
            for (int i = 0; i < k; ++i)
              for (int j = 0; j < k; ++j) {
                const int r = t.tm * k + i, c = t.tn * k + j;
                if (st < 2 && (t.tm > t.tn || r > c)) continue;   // mirrored cells are not computed
                if (r < 0 || c < 0 || r >= R || c >= W) {
                  std::printf("%s group %zu stage %d: cell (%d, %d) outside %d x %d\n", what, gi, st, r, c, R, W);
                  return 8;
                }
                ++cnt[((size_t)t.b * R + r) * W + c];
              }
          }
      for (int b = 0; b < g.n; ++b)
        for (int r = 0; r < R; ++r)
          for (int c = st < 2 ? r : 0; c < W; ++c)
            if (cnt[((size_t)b * R + r) * W + c] != 1) {
              std::printf("%s group %zu stage %d unit %d: cell (%d, %d) covered %d times\n", what, gi, st, b, r, c,
                          cnt[((size_t)b * R + r) * W + c]);
              return 9;
            }
    }
  }
  return 0;
}

// The elementwise work tables, for roots small enough to mark element by element:
// f0 tiles cover each Muon unit's padded layout once and sit in its group's lane
// range; AdamW segments cover the AdamW units' elements once (aseg_all), and so
// do the unfused segments together with the fused requant chunks' [lo, hi);
// requant chunks cover every quantised region once, fused chunks first.
int check_elementwise(const sshdp_plan &p, const std::vector<sshdp_node> &nodes, const char *what) {
  for (const sshdp::MuonUnit &u : p.munits) {
    const int TR = u.Rp / sshdp::kF0Tile, TC = u.Cp / sshdp::kF0Tile;
    std::vector<int> seen((size_t)TR * TC, 0);
    const int ln = p.group_lane[u.group];
    if (u.tile_begin < p.f0_lane[ln] || u.tile_end > p.f0_lane[ln + 1]) {
      std::printf("%s: unit's f0 tiles outside its lane's range\n", what);
      return 10;
    }
    for (int k = u.tile_begin; k < u.tile_end; ++k) {
      const sshdp::F0Tile &t = p.f0tiles[k];
      if (&p.munits[t.unit] != &u || t.tr < 0 || t.tr >= TR || t.tc < 0 || t.tc >= TC) {
        std::printf("%s: f0 tile %d does not belong to its unit\n", what, k);
        return 10;
      }
      ++seen[(size_t)t.tr * TC + t.tc];
    }
    for (int v : seen)
      if (v != 1) {
        std::printf("%s: an f0 tile covered %d times\n", what, v);
        return 10;
      }
  }
  if (p.root_numel > ((int64_t)1 << 27)) return 0;
  const size_t N = (size_t)p.root_numel;
  std::vector<uint8_t> want(N, 0), all(N, 0), upd(N, 0), quant(N, 0), qwant(N, 0);
  for (size_t i = 0; i < nodes.size(); ++i) {
    const sshdp_node &nd = nodes[i];
    if (!nd.is_unit || nd.optimizer != SSHDP_OPT_ADAMW) continue;
    const int64_t rs = nd.rows > 1 ? nd.row_stride : nd.cols;
    for (int64_t r = 0; r < nd.rows; ++r)
      for (int64_t c = 0; c < nd.cols; ++c) want[p.node_abs[i] + r * rs + c] = 1;
  }
  for (const sshdp::ASeg &g : p.aseg_all)
    for (int64_t e = g.base; e < g.base + g.n; ++e) ++all[e];
  for (const sshdp::ASeg &g : p.aseg_unfused)
    for (int64_t e = g.base; e < g.base + g.n; ++e) ++upd[e];
  for (size_t k = 0; k < p.qchunks.size(); ++k) {
    const sshdp::QChunk &q = p.qchunks[k];
    const sshdp::QRegion &rg = p.qregions[q.region];
    const int64_t end = rg.abs + rg.rows * rg.cols;
    const bool fused = (int64_t)k < p.n_qchunks_fused;
    if (q.n <= 0 || q.n % 32 || q.base < rg.abs || q.base + q.n > end || q.lo < q.base || q.hi < q.lo ||
        q.hi > q.base + q.n || (!fused && q.hi != q.lo) || q.row0 != (q.base - rg.abs) / rg.cols ||
        q.col0 != (q.base - rg.abs) % rg.cols) {
      std::printf("%s: requant chunk %zu malformed\n", what, k);
      return 11;
    }
    for (int64_t e = q.base; e < q.base + q.n; ++e) ++quant[e];
    for (int64_t e = q.lo; e < q.hi; ++e) ++upd[e];
  }
  for (const sshdp::QRegion &rg : p.qregions)
    for (int64_t e = rg.abs; e < rg.abs + rg.rows * rg.cols; ++e) ++qwant[e];
  for (size_t e = 0; e < N; ++e) {
    if (all[e] != want[e] || upd[e] != want[e] || quant[e] != qwant[e] || qwant[e] > 1) {
      std::printf("%s: element %zu: AdamW unit %d, segments %d, updated %d times, quantised %d (regions %d)\n", what,
                  e, want[e], all[e], upd[e], quant[e], qwant[e]);
      return 12;
    }
  }
  return 0;
}

int tiles_mode(const char *path) {
  FILE *f = std::fopen(path, "rb");
  if (!f) return 2;
  int trees = 0, plans = 0;
  for (;; ++trees) {
    int32_t n = 0, layout = 0;
    int64_t root = 0;
    uint32_t flags = 0;
    if (std::fread(&n, 4, 1, f) != 1) break;
    if (std::fread(&root, 8, 1, f) != 1 || std::fread(&layout, 4, 1, f) != 1 || std::fread(&flags, 4, 1, f) != 1 ||
        n <= 0)
      return 3;
    std::vector<sshdp_node> nodes(n);
    if (std::fread(nodes.data(), sizeof(sshdp_node), n, f) != (size_t)n) return 3;
    const uint32_t policies[] = {0, SSHDP_PLAN_NS_TILES_SMALL, SSHDP_PLAN_NS_TILES_LARGE, SSHDP_PLAN_NS_GRAM_NT,
                                 SSHDP_PLAN_NS_ONE_STREAM};
    for (uint32_t pol : policies) {
      sshdp_plan_opts o;
      sshdp_default_opts(&o);
      o.scale_layout = layout;
      o.flags = flags | pol | SSHDP_PLAN_HOST_ONLY;
      sshdp_plan *p = nullptr;
      if (sshdp_plan_views(nodes.data(), n, root, &o, &p) != SSHDP_OK) continue;   // rejected trees have no tiles
      // TILECHK_PLANT=drop|dup plants a mistake in the first non-empty tile table,
      // =seg doubles the first AdamW segment a step runs (or the first fused
      // requant chunk), to show the checks see a missing or a doubled item
      const char *plant = std::getenv("TILECHK_PLANT");
      const bool plant_seg = plant && std::strcmp(plant, "seg") == 0;
      if (plant_seg) {
        if (!p->aseg_unfused.empty()) {
          p->aseg_unfused.push_back(p->aseg_unfused.front());
        } else if (p->n_qchunks_fused > 0) {
          p->qchunks.insert(p->qchunks.begin(), p->qchunks.front());
          ++p->n_qchunks_fused;
        }
      } else if (plant) {
        bool done = false;
        for (int ln = 0; ln < sshdp::kMaxLanes && !done; ++ln)
          for (int st = 0; st < 3 && !done; ++st)
            for (int sz = 0; sz < 2 && !done; ++sz) {
              std::vector<sshdp::NsTile> &v = p->ns_tiles[ln][st][sz];
              if (v.empty()) continue;
              if (plant[0] == 'd' && plant[1] == 'r') v.pop_back();
              else v.push_back(v.front());
              done = true;
            }
      }
      char what[64];
      std::snprintf(what, sizeof what, "tree %d flags %u", trees, o.flags);
      int rc = plant_seg ? 0 : check_tiles(*p, what);
      if (!rc && (!plant || plant_seg)) rc = check_elementwise(*p, nodes, what);
      sshdp_plan_destroy(p);
      if (rc) return rc;
      ++plans;
    }
  }
  std::fclose(f);
  std::printf("ok trees %d plans %d\n", trees, plans);
  return 0;
}
}  // namespace

int main(int argc, char **argv) {
  if (argc == 3 && std::strcmp(argv[2], "tiles") == 0) return tiles_mode(argv[1]);
  if (argc != 2) return 2;
  FILE *f = std::fopen(argv[1], "rb");
  if (!f) return 2;
  int32_t n = 0, layout = 0;
  int64_t root = 0;
  uint32_t flags = 0;
  if (std::fread(&n, 4, 1, f) != 1 || std::fread(&root, 8, 1, f) != 1 || std::fread(&layout, 4, 1, f) != 1 ||
      std::fread(&flags, 4, 1, f) != 1 || n <= 0)
    return 3;
  std::vector<sshdp_node> nodes(n);
  if (std::fread(nodes.data(), sizeof(sshdp_node), n, f) != (size_t)n) return 3;
  std::fclose(f);
  sshdp_plan_opts o;
  sshdp_default_opts(&o);
  o.scale_layout = layout;
  o.flags = flags;
  sshdp_plan *p = nullptr;
  if (sshdp_plan_views(nodes.data(), n, root, &o, &p) != SSHDP_OK) return 4;
  sshdp_plan_stats st{};
  sshdp_plan_info(p, &st);
  // device roots are never dereferenced here: any 256-aligned address will do
  char *fake = reinterpret_cast<char *>(uintptr_t(1) << 40);
  sshdp_buffers b{};
  b.w_main = reinterpret_cast<float *>(fake);
  b.grad = reinterpret_cast<const float *>(fake + (1ll << 34));
  b.mom = reinterpret_cast<float *>(fake + (2ll << 34));
  b.adam_v = reinterpret_cast<float *>(fake + (3ll << 34));
  b.codes = reinterpret_cast<uint8_t *>(fake + (4ll << 34));
  b.scales = reinterpret_cast<uint8_t *>(fake + (5ll << 34));
  void *ws = fake + (6ll << 34);
  sshdp_muon_hp mh{0.02f, 0.95f, 0.f};
  sshdp_adamw_hp ah{1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f};
  hipStream_t caller = nullptr;
  hipStreamCreateWithFlags(&caller, 0);
  int lanes_seen = 0, checked = 0, launches = -1;
  for (int fail_at = 1;; ++fail_at) {
    for (int call = 0; call < 2; ++call) {        // the whole step, and Muon alone
      g_log.clear();
      g_launch = 0;
      g_fail_at = fail_at;
      const int rc = call == 0 ? sshdp_update_step(p, &b, &mh, &ah, 1, ws, (size_t)st.workspace_bytes, caller)
                               : sshdp_update_muon(p, &b, &mh, ws, (size_t)st.workspace_bytes, caller);
      const bool failed = g_launch >= fail_at;
      if (failed ? rc != SSHDP_ERR_HIP : rc != SSHDP_OK) {
        std::printf("call %d fail_at %d: status %d after %d launches\n", call, fail_at, rc, g_launch);
        return 5;
      }
      int bad = -1;
      if (!joined(caller->id, &bad)) {
        std::printf("call %d fail_at %d: side stream %d not joined into the caller's stream\n", call, fail_at, bad);
        return 6;
      }
      int side = 0;
      for (const Op &op : g_log) side = op.stream != caller->id ? 1 : side;
      lanes_seen |= side;
      ++checked;
      if (call == 0 && !failed) launches = g_launch;
    }
    if (launches >= 0) break;                      // fail_at passed the launches of a whole step
  }
  std::printf("ok checked %d launches_per_step %d side_streams %d\n", checked, launches, lanes_seen);
  sshdp_plan_destroy(p);
  hipStreamDestroy(caller);
  return 0;
}
