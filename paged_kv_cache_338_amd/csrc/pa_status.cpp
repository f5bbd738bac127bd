// Status names and the thread-local last-error text of the C ABI.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace pa {

pa_status fail(pa_status status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

}  // namespace pa

extern "C" {

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
    case PA_ERR_UNKNOWN_SEQ: return "PA_ERR_UNKNOWN_SEQ";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_DEVICE: return "PA_ERR_DEVICE";
    default: return "PA_UNKNOWN_STATUS";
  }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
