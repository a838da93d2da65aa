// Internal: per-thread error message and debug switch shared by every part of
// the library. Plain C++ (no HIP), so the host allocator builds with g++ alone.
#pragma once

#include "pagedkv.h"

namespace pagedkv {

// Record `msg` (printf-style) as the calling thread's last error; returns code.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the calling thread's last error.
void clear_error();
// True when the environment variable PA_DEBUG is set to a non-zero value
// (read at every call, so a process can switch it on and off).
bool debug_enabled();

}  // namespace pagedkv
