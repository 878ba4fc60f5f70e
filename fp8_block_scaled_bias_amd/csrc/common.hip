// Error state and version of libmoe_fp8.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace moe {

static thread_local char g_err[512] = {0};

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = 0; }

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: HIP launch failed: %s", what, hipGetErrorString(e));
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

}  // namespace moe

extern "C" const char* moe_last_error(void) { return moe::g_err; }

extern "C" const char* moe_version(void) { return "moe_fp8 0.1 gfx950"; }
