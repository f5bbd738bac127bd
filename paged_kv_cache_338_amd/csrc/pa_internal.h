// Internal helpers shared by the library's translation units (not installed).
#pragma once

#include "pa.h"

namespace pa {

// Records a printf-style message as the calling thread's last error and
// returns `status`, so callers can write `return fail(PA_ERR_..., "...")`.
pa_status fail(pa_status status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// log2 of x if x is a power of two >= 1, else -1.
int ilog2_exact(int32_t x);

// Bytes per stored value of a pool dtype.
inline int elem_bytes(pa_dtype d) { return d == PA_F32 ? 4 : 2; }

// Validates a pool descriptor against the supported set (see pa.h).
pa_status check_desc(const pa_cache_desc* desc);

// Current value of a process-wide tuning knob (0 = automatic); see
// pa_set_tuning.
int32_t tuning(pa_tuning_key key);

// True if p is a multiple of `bytes` (a power of two).
inline bool aligned(const void* p, uintptr_t bytes) {
  return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0;
}

}  // namespace pa
