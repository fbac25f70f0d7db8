// Error reporting and version query of the kvc C ABI.
#include <stdarg.h>
#include <stdio.h>

#include "common.hpp"

namespace kvc {

namespace {
thread_local std::string g_last_error;
}

kvc_status fail(kvc_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

kvc_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return KVC_OK;
}

}  // namespace kvc

extern "C" const char* kvc_last_error(void) { return kvc::g_last_error.c_str(); }

extern "C" int kvc_version(void) { return 100; }  // 0.1.0
