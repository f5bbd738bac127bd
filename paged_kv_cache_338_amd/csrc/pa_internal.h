// Internal helpers shared by the library's translation units (not installed).
#pragma once

#include "pa.h"

namespace pa {

// Records a printf-style message as the calling thread's last error and
// returns `status`, so callers can write `return fail(PA_ERR_..., "...")`.
pa_status fail(pa_status status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pa
