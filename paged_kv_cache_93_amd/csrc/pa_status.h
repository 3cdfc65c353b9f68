// Status reporting shared by every libpagedattn source, HIP or host-only.
#pragma once

#include "pagedattn.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace pa {

// Records a formatted message for pa_last_error() and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pa
