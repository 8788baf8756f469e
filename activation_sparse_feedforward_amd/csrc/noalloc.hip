// Allocation-free hybrid forward: twell_ffn_fwd_hybrid with its workspace in a
// static device array instead of a caller-provided buffer, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The array below has one copy per device, created when the code object is
// loaded on that device and held until the process ends.  In host code its
// name is only a host-side stand-in: the device address of each device's copy
// is looked up once per device with hipGetSymbolAddress (that device current)
// and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/twell.h"
#include "api_internal.hpp"

namespace {

__device__ __align__(256) char scratch[TWELL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of the current device's copy of `scratch`.  Two threads may
// both look it up on a device's first call; they store the same address.
twell_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TWELL_EHIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TWELL_EHIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return TWELL_OK;
}

}  // namespace

extern "C" twell_status twell_ffn_fwd_hybrid_noalloc(const twell_desc* d, const void* x, const void* w_gate_t,
                                                     twell_act act, const void* w_up_t, const void* w_down,
                                                     void* y, const twell_route* route, void* stream) {
  size_t need = 0;
  const twell_status st = twell::hybrid_check(d, x, w_gate_t, act, w_up_t, w_down, y, route, &need);
  if (st != TWELL_OK) return st;
  if (d->T == 0) return TWELL_OK;
  if (need > TWELL_NOALLOC_SCRATCH_BYTES) return TWELL_ESCRATCH;
  void* ws = nullptr;
  const twell_status sa = scratch_address(&ws);
  if (sa != TWELL_OK) return sa;
  return twell::hybrid_launch(d, x, w_gate_t, act, w_up_t, w_down, y, route, ws, stream);
}
