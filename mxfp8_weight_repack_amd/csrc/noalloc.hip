// noalloc.hip -- sshdp_update_step for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc): the step's workspace is a file-scope device array of fixed size
// instead of caller memory.
//
// The array lives in the code object, so every GPU the library is loaded on
// holds its own copy from module load until the process ends.  Host code never
// passes the array's name to a kernel (in host code it is a stand-in, not a
// device address): the first call on a device, with that device current, asks
// the runtime for the array's address on it and keeps it per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // SSHDP_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == SSHDP_NOALLOC_SCRATCH_BYTES, "header and library agree on the scratch size");
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// The array's address on `dev` (current), looked up once per device.
int scratch_ptr(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return SSHDP_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSHDP_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return SSHDP_OK;
}

}  // namespace

extern "C" int sshdp_update_step_noalloc(const sshdp_plan *p, const sshdp_buffers *b, const sshdp_muon_hp *mh,
                                         const sshdp_adamw_hp *ah, int64_t step, void *stream) {
  if (!p) return SSHDP_ERR_ARG;
  if (p->host_only) return SSHDP_ERR_STATE;
  if (p->ws_bytes > kScratchBytes) return SSHDP_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SSHDP_ERR_HIP;
  if (dev != p->device) return SSHDP_ERR_ARG;
  void *ws = nullptr;
  const int st = scratch_ptr(dev, &ws);
  if (st != SSHDP_OK) return st;
  return sshdp_update_step(p, b, mh, ah, step, ws, kScratchBytes, stream);
}
