// Error state of libmoe.so: every entry point that fails leaves a message for moe_last_error()
// in a thread-local buffer and returns its moe_status.
#include <stdarg.h>
#include <stdio.h>

#include "common.hpp"

namespace moe {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) { return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e)); }

}  // namespace moe

extern "C" const char* moe_last_error(void) { return moe::g_err; }
