// Status names, the thread-local last-error text and the shape checks of
// the C ABI (host code).
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

int ilog2_exact(int32_t x) {
  if (x < 1 || (x & (x - 1))) return -1;
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

pa_status check_desc(const pa_cache_desc* desc) {
  if (!desc) return fail(PA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (desc->num_blocks < 1 || desc->num_kv_heads < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks %d / num_kv_heads %d must be >= 1",
                desc->num_blocks, desc->num_kv_heads);
  const int lg = ilog2_exact(desc->block_size);
  if (lg < 0 || lg > 8)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d is not a power of two in [1, 256]",
                desc->block_size);
  if (desc->head_dim != 64 && desc->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", desc->head_dim);
  if (desc->dtype != PA_F32 && desc->dtype != PA_BF16 && desc->dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "dtype %d not in {PA_F32, PA_BF16, PA_F16}", desc->dtype);
  return PA_OK;
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
