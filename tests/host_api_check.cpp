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
}  // namespace

int main(int argc, char **argv) {
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
