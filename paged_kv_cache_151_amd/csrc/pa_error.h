// Thread-local error reporting shared by the library's C-ABI entry points.
#pragma once

#include "pa.h"

namespace pa {

// Records a formatted detail for pa_last_error() and returns `st`.
pa_status fail(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the detail and returns PA_OK.
pa_status ok();

}  // namespace pa
