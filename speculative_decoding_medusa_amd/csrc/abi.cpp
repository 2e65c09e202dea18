// Status strings, per-thread error text and the ABI version.
#include <stdarg.h>
#include <stdio.h>

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace {
thread_local char g_last_error[512] = "";
}

namespace medusa_host {

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

int hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return MEDUSA_ERR_HIP;
  }
  g_last_error[0] = '\0';
  return MEDUSA_OK;
}

}  // namespace medusa_host

extern "C" const char* medusa_status_string(int status) {
  switch (status) {
    case MEDUSA_OK: return "ok";
    case MEDUSA_ERR_NULL: return "null pointer";
    case MEDUSA_ERR_SHAPE: return "unsupported shape";
    case MEDUSA_ERR_DTYPE: return "unsupported dtype";
    case MEDUSA_ERR_VALUE: return "argument out of range";
    case MEDUSA_ERR_WORKSPACE: return "workspace too small";
    case MEDUSA_ERR_HIP: return "HIP launch failed";
    case MEDUSA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MEDUSA_ERR_ALIAS: return "output aliases an input";
    default: return "unknown status";
  }
}

extern "C" const char* medusa_last_error(void) { return g_last_error; }

extern "C" int medusa_abi_version(void) { return 109; }
