// Per-thread error state and the PA_DEBUG switch.
#include "status.h"

#include <cstdarg>
#include <cstdio>
#include <cstdlib>

namespace pagedkv {

namespace {
thread_local char g_last_error[512] = "";
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_last_error[0] = '\0'; }

bool debug_enabled() {
  const char* v = std::getenv("PA_DEBUG");
  return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
}

}  // namespace pagedkv

extern "C" const char* pa_last_error(void) { return pagedkv::g_last_error; }
