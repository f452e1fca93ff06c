// Internal hooks of the optional per-kernel launch timing (timing.cpp).
#pragma once

#include <hip/hip_runtime.h>

namespace cartattn {

// Returns a slot (or -1 when timing is off); pass it to timing_stop after the
// launch. `name` must be a string literal.
int timing_start(const char* name, hipStream_t st);
void timing_stop(int slot, hipStream_t st);

// Launch the statement (a kernel launch) between the two timing events of `name`.
#define CART_TIMED(name, st, ...)                         \
  do {                                                    \
    const int _slot = ::cartattn::timing_start(name, st); \
    __VA_ARGS__;                                          \
    ::cartattn::timing_stop(_slot, st);                   \
  } while (0)

}  // namespace cartattn
