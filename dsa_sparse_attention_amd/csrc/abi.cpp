// abi.cpp -- version and error plumbing of the C ABI (host only).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>

#include "common.hpp"

namespace dsa {

static thread_local char g_last_error[512] = "";

dsa_status fail(dsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

dsa_status ok() {
  g_last_error[0] = '\0';
  return DSA_OK;
}

dsa_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace dsa

extern "C" int dsa_abi_version(void) { return DSA_ABI_VERSION; }

extern "C" const char* dsa_last_error(void) { return dsa::g_last_error; }
