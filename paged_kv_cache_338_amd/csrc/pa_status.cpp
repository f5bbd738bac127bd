// Status names, the thread-local last-error text and the shape checks of
// the C ABI (host code).
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa_internal.h"

namespace {
thread_local std::string g_last_error;
// Tuning knobs, indexed by pa_tuning_key; 0 = the library's own choice.
std::atomic<int32_t> g_tuning[4];
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

int32_t tuning(pa_tuning_key key) {
  return key >= 1 && key <= 3 ? g_tuning[key].load(std::memory_order_relaxed) : 0;
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

pa_status pa_set_tuning(pa_tuning_key key, int32_t value) {
  switch (key) {
    case PA_TUNE_DECODE_WORKGROUPS:
      if (value < 0 || value > 1024)
        return pa::fail(PA_ERR_INVALID_ARGUMENT, "decode workgroups %d not in [0, 1024]", value);
      break;
    case PA_TUNE_PREFILL_KEY_TILES:
      if (value < 0 || value > (1 << 20))
        return pa::fail(PA_ERR_INVALID_ARGUMENT, "prefill key tiles %d not in [0, 2^20]", value);
      break;
    case PA_TUNE_DECODE_KV_CACHED:
      if (value < 0 || value > 1)
        return pa::fail(PA_ERR_INVALID_ARGUMENT, "decode KV cached %d not 0 or 1", value);
      break;
    default:
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "unknown tuning key %d", key);
  }
  g_tuning[key].store(value, std::memory_order_relaxed);
  return PA_OK;
}

pa_status pa_get_tuning(pa_tuning_key key, int32_t* value) {
  if (!value) return pa::fail(PA_ERR_INVALID_ARGUMENT, "value is NULL");
  if (key != PA_TUNE_DECODE_WORKGROUPS && key != PA_TUNE_PREFILL_KEY_TILES &&
      key != PA_TUNE_DECODE_KV_CACHED)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "unknown tuning key %d", key);
  *value = pa::tuning(key);
  return PA_OK;
}

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
