// Internal hooks of the optional per-kernel launch timing (timing.cpp).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace cartattn {

// Events for one launch of kernel `name` (a string literal): both set when
// this launch is timed, both null otherwise.
void timing_events(const char* name, hipEvent_t* start, hipEvent_t* stop);

// Launch `kernel` (parenthesised when it is a template id with commas) with
// the given grid, block, dynamic LDS bytes, stream and arguments. A timed
// launch carries its two events in the dispatch itself (hipExtLaunchKernel),
// so timing adds no separate marker packets between kernels.
#define CART_LAUNCH(name, kernel, grid, block, shmem, st, ...)                          \
  do {                                                                                  \
    hipEvent_t _e0 = nullptr, _e1 = nullptr;                                            \
    ::cartattn::timing_events(name, &_e0, &_e1);                                        \
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), shmem, st, _e0, _e1, 0u,     \
                          __VA_ARGS__);                                                 \
  } while (0)

}  // namespace cartattn
