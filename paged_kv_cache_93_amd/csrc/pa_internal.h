// Host-side helpers shared by the libpagedattn entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>

#include "pa_status.h"
#include "pagedattn.h"

namespace pa {

// Checks hipGetLastError() after a launch; PA_OK or PA_ERR_LAUNCH.
int launch_result(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int element_bytes(int32_t dtype) {
  return dtype == PA_F32 ? 4 : dtype == PA_BF16 ? 2 : dtype == PA_FP8_E4M3 ? 1 : 0;
}

// Validates the pool description shared by every cache entry point.
int check_cache(const pa_cache* cache, const char* fn);

// A pointer argument and its name, for check_device_memory.
struct NamedPtr {
  const char* name;
  const void* ptr;
};

// PA_OK when every non-NULL pointer in `ptrs` is device memory of the current
// device or managed memory, as the HIP runtime reports it; otherwise
// PA_ERR_SHAPE naming the first that is not.  A plain host pointer handed to
// a kernel would fault the GPU, so every entry point calls this after its
// other checks and before it enqueues anything.
int check_device_memory(const char* fn, std::initializer_list<NamedPtr> ptrs);

}  // namespace pa
