// api.hip -- the launching entry points of libsshdp.so.
//
// [SS-HSDP §3.4 "Update"]: once the microbatches are done, every unit runs
// its F (for Muon: f0 on local momentum, f1 Newton-Schulz over the whole
// unit, f2 on the local weight), the remaining units take AdamW, and G then
// turns the new main weights into the next iteration's runtime weights.
// [SS-HSDP Appendix A]: within an update group the stages are ordered, each
// reading what the previous one committed; here that order is the order of
// launches on one stream.
//
// This file launches no kernel itself (the launchers live beside their
// kernels), so it needs only the runtime API.
#include <hip/hip_runtime_api.h>

#include "internal.h"

using namespace sshdp;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? SSHDP_OK : SSHDP_ERR_HIP; }

int check_plan(const sshdp_plan *p) {
  if (!p) return SSHDP_ERR_ARG;
  if (p->host_only) return SSHDP_ERR_STATE;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return SSHDP_ERR_HIP;
  if (cur != p->device) return SSHDP_ERR_ARG;
  return SSHDP_OK;
}

// Event bracketing of one kernel class (measurement only).
struct Prof {
  sshdp_plan *p;
  int cls;
  hipStream_t s;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  Prof(const sshdp_plan *pl, int c, hipStream_t st) : p(const_cast<sshdp_plan *>(pl)), cls(c), s(st) {
    if (!p->prof || cls < 0) return;
    e0 = take();
    e1 = take();
    if (e0) (void)hipEventRecord(e0, s);
  }
  ~Prof() {
    if (!p->prof || cls < 0 || !e0 || !e1) return;
    (void)hipEventRecord(e1, s);
    p->prof_pending.push_back({cls, {e0, e1}});
  }
  hipEvent_t take() {
    if (!p->prof_pool.empty()) {
      hipEvent_t e = p->prof_pool.back();
      p->prof_pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

// The plan's side streams (lanes 1..) forked from the caller's stream by an event.
// Every lane that has started waiting on the fork is joined back into the caller's
// stream -- explicitly on success, by the destructor on an error return -- so a call
// that fails part-way still leaves no side-stream work unordered after the caller's
// later work (and a capture that began on the caller's stream stays closed).
struct LaneFork {
  const sshdp_plan *p;
  hipStream_t s;
  int forked = 1;        // lanes [1, forked) wait on the fork
  LaneFork(const sshdp_plan *pl, hipStream_t st) : p(pl), s(st) {}
  hipError_t fork() {
    hipError_t e = hipEventRecord(p->ev_fork, s);
    for (int ln = 1; e == hipSuccess && ln < p->n_lanes; ++ln) {
      e = hipStreamWaitEvent(p->lane_stream[ln], p->ev_fork, 0);
      if (e == hipSuccess) forked = ln + 1;
    }
    return e;
  }
  hipError_t join() {
    hipError_t first = hipSuccess;
    for (int ln = 1; ln < forked; ++ln) {
      hipError_t e = hipEventRecord(p->ev_join[ln], p->lane_stream[ln]);
      if (e == hipSuccess) e = hipStreamWaitEvent(s, p->ev_join[ln], 0);
      if (e != hipSuccess && first == hipSuccess) first = e;
    }
    forked = 1;
    return first;
  }
  ~LaneFork() { (void)join(); }
};

// side_adam: the step's unfused AdamW units, run on the last side stream after its
// Newton-Schulz work (AdamW and Muon units are disjoint; G waits for the join), so they
// leave the caller's stream; with one stream they are the caller's to launch.
int run_muon(const sshdp_plan *p, const sshdp_buffers *b, const sshdp_muon_hp *hp, void *ws, size_t ws_bytes,
             hipStream_t s, const sshdp_adamw_hp *side_adam = nullptr, int64_t step = 0, bool *adam_done = nullptr) {
  if (p->munits.empty()) return SSHDP_OK;
  if (!b->w_main || !b->grad || !b->mom) return SSHDP_ERR_ARG;
  if (!aligned16(b->w_main) || !aligned16(b->grad) || !aligned16(b->mom)) return SSHDP_ERR_ALIGN;
  if (!ws || ws_bytes < p->ws_bytes) return SSHDP_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) return SSHDP_ERR_ALIGN;
  char *w = static_cast<char *>(ws);
  hipError_t e;
  // lane 0 (the caller's stream): f0 and the norms of its own units; the side lanes,
  // forked after that, run their f0 and norms beside lane 0's first Gram
  {
    Prof pr(p, 0, s);
    e = launch_f0(*p, 0, b->grad, b->mom, hp->momentum, p->opts.nesterov, w, s);
  }
  if (e != hipSuccess) return SSHDP_ERR_HIP;
  {
    Prof pr(p, 1, s);
    e = launch_norm(*p, 0, w, p->opts.ns_eps, s);
  }
  if (e != hipSuccess) return SSHDP_ERR_HIP;
  // Newton-Schulz: lane 0 on the caller's stream, the other lanes on plan-owned
  // streams forked from and joined back into it by events
  Prof wall(p, 8, s);
  LaneFork lanes(p, s);
  if (p->n_lanes > 1) {
    if (lanes.fork() != hipSuccess) return SSHDP_ERR_HIP;
    for (int ln = 1; ln < p->n_lanes; ++ln) {
      hipStream_t ls = p->lane_stream[ln];
      {
        Prof pr(p, 0, ls);
        e = launch_f0(*p, ln, b->grad, b->mom, hp->momentum, p->opts.nesterov, w, ls);
      }
      if (e != hipSuccess) return SSHDP_ERR_HIP;
      Prof pr(p, 1, ls);
      if (launch_norm(*p, ln, w, p->opts.ns_eps, ls) != hipSuccess) return SSHDP_ERR_HIP;
    }
  }
  const int steps = p->opts.ns_steps;
  for (int it = 0; it < steps; ++it) {
    for (int stage = 0; stage < 3; ++stage) {
      const int kind = stage < 2 ? stage : (it + 1 == steps ? 3 : 2);
      for (int ln = 0; ln < p->n_lanes; ++ln) {
        hipStream_t ls = ln == 0 ? s : p->lane_stream[ln];
        Prof pr(p, 2 + stage, ls);
        if (ln == 0 && p->prof) {
          // the caller's stream's launches alone: Gram and poly per stage, the update's
          // 256-tile launch on its own (then its 128-tile launch, untimed)
          if (kind < 2) {
            Prof pr0(p, 10 + kind, ls);
            e = launch_ns_stage(*p, ln, kind, it, w, b->w_main, hp->lr, hp->weight_decay, ls);
          } else {
            {
              Prof pr0(p, 10 + kind, ls);
              e = launch_ns_stage(*p, ln, kind, it, w, b->w_main, hp->lr, hp->weight_decay, ls, 1);
            }
            if (e == hipSuccess) e = launch_ns_stage(*p, ln, kind, it, w, b->w_main, hp->lr, hp->weight_decay, ls, 2);
          }
        } else {
          e = launch_ns_stage(*p, ln, kind, it, w, b->w_main, hp->lr, hp->weight_decay, ls);
        }
        if (e != hipSuccess) return SSHDP_ERR_HIP;
      }
    }
  }
  if (p->n_lanes > 1 && side_adam && !p->aseg_unfused.empty()) {
    hipStream_t ls = p->lane_stream[p->n_lanes - 1];
    Prof pr(p, 5, ls);
    if (launch_adamw(p->d.aseg_unfused, (int64_t)p->aseg_unfused.size(), *b, *side_adam, step, ls) != hipSuccess)
      return SSHDP_ERR_HIP;
    if (adam_done) *adam_done = true;
  }
  return lanes.join() == hipSuccess ? SSHDP_OK : SSHDP_ERR_HIP;
}

int check_adam(const sshdp_plan *p, const sshdp_buffers *b, const sshdp_adamw_hp *hp, int64_t step) {
  if (!hp || step < 1) return SSHDP_ERR_ARG;
  if (!b->w_main || !b->grad || !b->mom || !b->adam_v) return SSHDP_ERR_ARG;
  if (!aligned16(b->w_main) || !aligned16(b->grad) || !aligned16(b->mom) || !aligned16(b->adam_v))
    return SSHDP_ERR_ALIGN;
  (void)p;
  return SSHDP_OK;
}

int check_quant(const float *w, const uint8_t *codes, const uint8_t *scales) {
  if (!w || !codes || !scales) return SSHDP_ERR_ARG;
  if (!aligned16(w) || !aligned16(codes)) return SSHDP_ERR_ALIGN;
  return SSHDP_OK;
}

}  // namespace

extern "C" {

int sshdp_update_muon(const sshdp_plan *p, const sshdp_buffers *b, const sshdp_muon_hp *hp, void *ws,
                      size_t ws_bytes, void *stream) {
  int st = check_plan(p);
  if (st != SSHDP_OK) return st;
  if (!b || !hp) return SSHDP_ERR_ARG;
  return run_muon(p, b, hp, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

int sshdp_update_adamw(const sshdp_plan *p, const sshdp_buffers *b, const sshdp_adamw_hp *hp, int64_t step,
                       void *stream) {
  int st = check_plan(p);
  if (st != SSHDP_OK) return st;
  if (!b) return SSHDP_ERR_ARG;
  if (p->aseg_all.empty()) return (hp && step >= 1) ? SSHDP_OK : SSHDP_ERR_ARG;
  st = check_adam(p, b, hp, step);
  if (st != SSHDP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Prof pr(p, 5, s);
  return hip_status(launch_adamw(p->d.aseg_all, (int64_t)p->aseg_all.size(), *b, *hp, step, s));
}

int sshdp_requant_mxfp8(const sshdp_plan *p, const float *w_main, uint8_t *codes, uint8_t *scales, void *stream) {
  int st = check_plan(p);
  if (st != SSHDP_OK) return st;
  if (p->qchunks.empty() && p->q32tiles.empty()) return SSHDP_OK;
  st = check_quant(w_main, codes, scales);
  if (st != SSHDP_OK) return st;
  sshdp_buffers b{};
  b.w_main = const_cast<float *>(w_main);
  b.codes = codes;
  b.scales = scales;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Prof pr(p, 7, s);
  if (!p->q32tiles.empty()) return hip_status(launch_quant32(*p, w_main, codes, scales, s));
  return hip_status(launch_quant(*p, 0, (int64_t)p->qchunks.size(), false, b, nullptr, 1, s));
}

int sshdp_cast_bf16(const sshdp_plan *p, const float *w_main, uint16_t *w_bf16, void *stream) {
  int st = check_plan(p);
  if (st != SSHDP_OK) return st;
  if (p->cchunks.empty()) return SSHDP_OK;
  if (!w_main || !w_bf16) return SSHDP_ERR_ARG;
  if (!aligned16(w_main) || !aligned16(w_bf16)) return SSHDP_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Prof pr(p, 9, s);
  return hip_status(launch_cast_bf16(*p, w_main, w_bf16, s));
}

namespace {
int rs_check(const void *const *inputs, int32_t n_inputs, int32_t in_dtype, const void *out, int64_t n, int64_t g0) {
  if (!inputs || !out || n_inputs < 1 || n_inputs > sshdp::kRsMaxInputs || n < 0) return SSHDP_ERR_ARG;
  if (in_dtype != SSHDP_RS_FP32 && in_dtype != SSHDP_RS_BF16) return SSHDP_ERR_ARG;
  for (int k = 0; k < n_inputs; ++k) {
    if (!inputs[k]) return SSHDP_ERR_ARG;
    if (!aligned16(inputs[k])) return SSHDP_ERR_ALIGN;
  }
  if (!aligned16(out)) return SSHDP_ERR_ALIGN;
  if (n % 16 || g0 % 16 || g0 < 0) return SSHDP_ERR_SCHEMA;
  return SSHDP_OK;
}
}  // namespace

int sshdp_rs_reduce(const void *const *inputs, int32_t n_inputs, int32_t in_dtype, void *out, int32_t out_mode,
                    int64_t n, uint64_t seed, uint64_t ctr, int64_t g0, void *stream) {
  int st = rs_check(inputs, n_inputs, in_dtype, out, n, g0);
  if (st != SSHDP_OK) return st;
  if (out_mode != SSHDP_RS_OUT_FP32 && out_mode != SSHDP_RS_OUT_BF16_SR) return SSHDP_ERR_ARG;
  if (n == 0) return SSHDP_OK;
  return hip_status(launch_rs_reduce(inputs, n_inputs, in_dtype == SSHDP_RS_BF16, out,
                                     out_mode == SSHDP_RS_OUT_BF16_SR, n, seed, ctr, g0,
                                     static_cast<hipStream_t>(stream)));
}

int sshdp_rs_accumulate(const void *const *inputs, int32_t n_inputs, int32_t in_dtype, float *g, int64_t n,
                        int32_t first, void *stream) {
  int st = rs_check(inputs, n_inputs, in_dtype, g, n, 0);
  if (st != SSHDP_OK) return st;
  if (n == 0) return SSHDP_OK;
  return hip_status(launch_rs_accumulate(inputs, n_inputs, in_dtype == SSHDP_RS_BF16, g, n, first != 0,
                                         static_cast<hipStream_t>(stream)));
}

int sshdp_update_step(const sshdp_plan *p, const sshdp_buffers *b, const sshdp_muon_hp *mh,
                      const sshdp_adamw_hp *ah, int64_t step, void *ws, size_t ws_bytes, void *stream) {
  int st = check_plan(p);
  if (st != SSHDP_OK) return st;
  if (!b) return SSHDP_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!p->munits.empty() && !mh) return SSHDP_ERR_ARG;
  if (!p->aseg_all.empty()) {
    st = check_adam(p, b, ah, step);
    if (st != SSHDP_OK) return st;
  } else if (step < 1) {
    return SSHDP_ERR_ARG;
  }
  if (!p->qchunks.empty() || !p->q32tiles.empty()) {
    st = check_quant(b->w_main, b->codes, b->scales);
    if (st != SSHDP_OK) return st;
  }
  if (!p->cchunks.empty()) {
    if (!b->w_main || !b->w_bf16) return SSHDP_ERR_ARG;
    if (!aligned16(b->w_main) || !aligned16(b->w_bf16)) return SSHDP_ERR_ALIGN;
  }
  bool adam_done = false;
  if (!p->munits.empty()) {
    st = run_muon(p, b, mh, ws, ws_bytes, s, ah, step, &adam_done);
    if (st != SSHDP_OK) return st;
  }
  if (!p->aseg_unfused.empty() && !adam_done) {
    Prof pr(p, 5, s);
    st = hip_status(launch_adamw(p->d.aseg_unfused, (int64_t)p->aseg_unfused.size(), *b, *ah, step, s));
  }
  if (st != SSHDP_OK) return st;
  if (p->n_qchunks_fused > 0) {
    if (!ah) return SSHDP_ERR_ARG;                 // fused chunks exist only beside AdamW units
    Prof pr(p, 6, s);
    st = hip_status(launch_quant(*p, 0, p->n_qchunks_fused, true, *b, ah, step, s));
  }
  if (st != SSHDP_OK) return st;
  const int64_t rest = (int64_t)p->qchunks.size() - p->n_qchunks_fused;
  if (rest > 0) {
    Prof pr(p, 7, s);
    st = hip_status(launch_quant(*p, p->n_qchunks_fused, rest, false, *b, nullptr, step, s));
  }
  if (st != SSHDP_OK) return st;
  if (!p->q32tiles.empty()) {
    Prof pr(p, 7, s);
    st = hip_status(launch_quant32(*p, b->w_main, b->codes, b->scales, s));
  }
  if (st != SSHDP_OK) return st;
  if (!p->cchunks.empty()) {
    Prof pr(p, 9, s);
    st = hip_status(launch_cast_bf16(*p, b->w_main, b->w_bf16, s));
  }
  return st;
}

int sshdp_gemm_bf16_nt(const void *P, const void *Q, const void *D, void *O, void *OT, int32_t M, int32_t N,
                       int32_t K, int32_t batch, float alpha, float beta, int32_t tile, void *stream) {
  if (!P || !Q || !O || M <= 0 || N <= 0 || K <= 0 || batch <= 0) return SSHDP_ERR_ARG;
  if (tile != 128 && tile != 256 && tile != 1281 && tile != 2561) return SSHDP_ERR_ARG;
  const int tt = tile == 1281 ? 128 : tile == 2561 ? 256 : tile;
  const bool kmajor = tile == 1281 || tile == 2561;
  if (M % tt || N % tt || K % 64) return SSHDP_ERR_SCHEMA;
  // each operand panel is one buffer resource with 32-bit byte offsets
  const int64_t span = !kmajor ? (int64_t)tt * K * 2 : ((int64_t)K - 1) * M * 2 + (int64_t)tt * 2;
  if (span > 0x7FFFFFFF) return SSHDP_ERR_SCHEMA;
  if (kmajor && (D || M != N)) return SSHDP_ERR_ARG;
  if (!aligned16(P) || !aligned16(Q) || (D && !aligned16(D)) || !aligned16(O) || (OT && !aligned16(OT)))
    return SSHDP_ERR_ALIGN;
  return hip_status(launch_gemm_raw(P, Q, D, O, OT, M, N, K, batch, alpha, D ? beta : 0.f, tile,
                                    static_cast<hipStream_t>(stream)));
}

int sshdp_ns_executed(const sshdp_plan *p, const void *ws, size_t ws_bytes, int32_t *units_per_group,
                      double *flops, void *stream) {
  int st = check_plan(p);
  if (st != SSHDP_OK) return st;
  if (flops) *flops = 0.0;
  for (size_t g = 0; units_per_group && g < p->groups.size(); ++g) units_per_group[g] = 0;
  if (p->munits.empty()) return SSHDP_OK;
  if (!ws || ws_bytes < p->ws_bytes) return SSHDP_ERR_WORKSPACE;
  std::vector<float> s(p->munits.size());
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(s.data(), static_cast<const char *>(ws) + p->ws_uscale, s.size() * sizeof(float),
                     hipMemcpyDeviceToHost, hs) != hipSuccess)
    return SSHDP_ERR_HIP;
  if (hipStreamSynchronize(hs) != hipSuccess) return SSHDP_ERR_HIP;
  double f = 0.0;
  for (size_t u = 0; u < s.size(); ++u) {
    if (s[u] == 0.0f) continue;
    const int g = p->munits[u].group;
    f += p->group_unit_flops[g];
    if (units_per_group) units_per_group[g] += 1;
  }
  if (flops) *flops = f;
  return SSHDP_OK;
}

int sshdp_profile_enable(sshdp_plan *p, int32_t enable) {
  if (!p) return SSHDP_ERR_ARG;
  p->prof = enable != 0;
  return SSHDP_OK;
}

int sshdp_profile_read(sshdp_plan *p, double *ms, int64_t *launches) {
  if (!p) return SSHDP_ERR_ARG;
  for (auto &e : p->prof_pending) {
    if (hipEventSynchronize(e.second.second) != hipSuccess) return SSHDP_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, e.second.first, e.second.second) != hipSuccess) return SSHDP_ERR_HIP;
    p->prof_ms[e.first] += t;
    p->prof_n[e.first] += 1;
    p->prof_pool.push_back(e.second.first);
    p->prof_pool.push_back(e.second.second);
  }
  p->prof_pending.clear();
  for (int i = 0; i < SSHDP_PROF_CLASSES; ++i) {
    if (ms) ms[i] = p->prof_ms[i];
    if (launches) launches[i] = p->prof_n[i];
    p->prof_ms[i] = 0.0;
    p->prof_n[i] = 0;
  }
  return SSHDP_OK;
}

}  // extern "C"
