// Status codes, per-thread error messages and the ABI version of libqlin.
#include <stdarg.h>
#include <stdio.h>

#include "common.hpp"

namespace qlin {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
}

qlin_status fail(qlin_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

qlin_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) return QLIN_OK;
  return fail(QLIN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace qlin

extern "C" int32_t qlin_abi_version(void) { return QLIN_ABI_VERSION; }

extern "C" const char* qlin_status_string(qlin_status s) {
  switch (s) {
    case QLIN_OK: return "QLIN_OK";
    case QLIN_ERR_INVALID_ARG: return "QLIN_ERR_INVALID_ARG";
    case QLIN_ERR_SHAPE: return "QLIN_ERR_SHAPE";
    case QLIN_ERR_ALIGN: return "QLIN_ERR_ALIGN";
    case QLIN_ERR_UNSUPPORTED: return "QLIN_ERR_UNSUPPORTED";
    case QLIN_ERR_HIP: return "QLIN_ERR_HIP";
    default: return "QLIN_ERR_UNKNOWN";
  }
}

extern "C" const char* qlin_last_error(void) { return qlin::g_last_error; }
