// muon_step_noalloc: the Muon step for callers that cannot allocate device memory (code under
// stream capture, tight serving loops, harnesses that forbid allocation).
//
// The kernels' scratch memory (the plan's workspace: the Newton-Schulz iterates X, A, B',
// norm partials and scales, row-equaliser sums) comes from the static device array below
// instead of a caller-provided buffer. Each device the library runs on holds its own copy of
// the array from module load until the process ends. In host code `scratch` names a host-side
// stand-in, not a device address, so its address on a device is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that pointer is passed on.
//
// Nothing in the scratch has to start at zero: every step writes each workspace element it
// later reads within the same call. Calls share their device's array, so calls that may
// overlap on one device (different streams, or unordered host threads) race with each other.
#include <mutex>

#include "muon.h"
#include "muon_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MUON_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on its first use on that device.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return muon::fail(MUON_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return muon::fail(MUON_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return muon::fail(MUON_ERR_HIP, "hipGetSymbolAddress of the static scratch failed on "
                        "device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MUON_OK;
}

}  // namespace

extern "C" int muon_step_noalloc(muon_plan* plan, const muon_matrix* mats, int64_t n,
                                 const muon_config* cfg, hipStream_t stream) {
  muon::clear_error();
  if (!plan) return muon::fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  const size_t need = muon_plan_workspace_size(plan);
  if (need > MUON_STATIC_SCRATCH_BYTES)
    return muon::fail(MUON_ERR_WORKSPACE,
                      "the plan needs %zu bytes of scratch; the static scratch of "
                      "muon_step_noalloc holds %zu (use muon_step with a workspace)",
                      need, (size_t)MUON_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0)
    if (int st = scratch_of_current_device(&ws)) return st;
  return muon_step(plan, mats, n, cfg, ws, need > 0 ? MUON_STATIC_SCRATCH_BYTES : 0, stream);
}
