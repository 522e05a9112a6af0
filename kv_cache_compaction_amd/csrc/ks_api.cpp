// Host-side plumbing of the libks C ABI: thread-local error message,
// launch checking and the version string.  The entry points themselves live
// next to their kernels.
#include <stdarg.h>
#include <stdio.h>

#include "ks_common.h"

static thread_local char g_err[512] = "";

ks_status ks_fail(ks_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ks_status ks_check_launch(const char* what) {
  hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return ks_fail(KS_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(err));
  return KS_OK;
}

extern "C" const char* ks_last_error(void) { return g_err; }

extern "C" const char* ks_version(void) { return "libks 0.1 (gfx950)"; }
