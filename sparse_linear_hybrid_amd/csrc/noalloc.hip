// Allocation-free entry point (include/sla.h, sla_forward_cached_noalloc): the cached
// (decode) forward with its workspace in a fixed device array of the library instead of a
// caller-supplied buffer, for callers that cannot allocate device memory. The kernels are
// those of sla_forward_cached; only where their scratch lives differs.
#include <mutex>

#include "common.h"
#include "kernels.h"

// The workspace of every call on a GPU: one copy per device, held from the code object's
// load until the process ends. Host code never uses this name as an address (on the host it
// is only a stand-in for the device symbol); it looks the device address up once per device
// with hipGetSymbolAddress and passes that pointer on.
static __device__ __align__(256) unsigned char scratch[SLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, or null

// Device address of the scratch array on the current device (looked up on the first call on
// that device, with the device current).
sla_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SLA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SLA_OK;
}

}  // namespace

extern "C" sla_status sla_forward_cached_noalloc(const sla_problem* p, const void* q,
                                                 const void* k, const void* v,
                                                 const float* proj_q, const float* alpha,
                                                 const void* cache, void* o,
                                                 int32_t* block_idx, hipStream_t stream) {
  const size_t need = sla_cached_workspace_size(p);
  if (need == 0)   // an invalid problem: the plain entry point says why and enqueues nothing
    return sla_forward_cached(p, q, k, v, proj_q, alpha, cache, o, block_idx, nullptr, 0, stream);
  if (need > SLA_NOALLOC_SCRATCH_BYTES) return SLA_ERR_SCRATCH;
  void* ws = nullptr;
  const sla_status st = scratch_address(&ws);
  if (st != SLA_OK) return st;
  return sla_forward_cached(p, q, k, v, proj_q, alpha, cache, o, block_idx, ws, need, stream);
}
