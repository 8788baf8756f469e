// Host-side pieces of the C-ABI layer shared by more than one entry point.
#pragma once

#include <stddef.h>

#include "../../include/twell.h"

namespace twell {

// The hybrid forward in two halves.  hybrid_check validates every argument
// except the workspace (no HIP call) and returns the workspace bytes the
// call needs in *ws_need (0 when d->T == 0, which is a no-op).
// hybrid_launch runs the kernels on checked arguments with a workspace of at
// least that many bytes, 16-byte aligned.
twell_status hybrid_check(const twell_desc* d, const void* x, const void* w_gate_t, twell_act act,
                          const void* w_up_t, const void* w_down, void* y, const twell_route* route,
                          size_t* ws_need);
twell_status hybrid_launch(const twell_desc* d, const void* x, const void* w_gate_t, twell_act act,
                           const void* w_up_t, const void* w_down, void* y, const twell_route* route,
                           void* ws, void* stream);

}  // namespace twell
