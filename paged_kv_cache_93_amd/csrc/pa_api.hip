// Library-wide entry points of libpagedattn: version queries, the per-thread
// error message, and the pool checks every cache entry point shares.
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "pa_internal.h"

#include <cstddef>

static_assert(sizeof(pa_cache) == 64 && offsetof(pa_cache, dtype) == 36 &&
                  offsetof(pa_cache, k_scale) == 40 && offsetof(pa_cache, v_scale) == 44 &&
                  offsetof(pa_cache, k_scales) == 48 && offsetof(pa_cache, v_scales) == 56,
              "pa_cache layout is part of the ABI");
static_assert(sizeof(pa_attn_variant) == 16 && offsetof(pa_attn_variant, alibi_slopes) == 8,
              "pa_attn_variant layout is part of the ABI");

namespace pa {

static thread_local char g_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return status;
}

int launch_result(const char* what) {
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    return fail(PA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(err));
  }
  return PA_OK;
}

int check_cache(const pa_cache* cache, const char* fn) {
  if (cache == nullptr) return fail(PA_ERR_NULL, "%s: cache is NULL", fn);
  if (cache->k_pool == nullptr || cache->v_pool == nullptr)
    return fail(PA_ERR_NULL, "%s: k_pool or v_pool is NULL", fn);
  if (element_bytes(cache->dtype) == 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: unknown cache dtype %d", fn, cache->dtype);
  if (cache->num_blocks <= 0 || cache->num_kv_heads <= 0 || cache->block_size <= 0 ||
      cache->head_dim <= 0)
    return fail(PA_ERR_SHAPE, "%s: pool sizes must be positive", fn);
  const int64_t row_bytes = int64_t(cache->head_dim) * element_bytes(cache->dtype);
  if (row_bytes % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim*element size must be a multiple of 16 bytes",
                fn);
  // the whole pool must be addressable with 64-bit byte offsets
  const double total = double(cache->num_blocks) * cache->num_kv_heads * cache->block_size *
                       double(row_bytes);
  if (total > 9.0e18) return fail(PA_ERR_SHAPE, "%s: pool too large", fn);
  if (!aligned16(cache->k_pool) || !aligned16(cache->v_pool))
    return fail(PA_ERR_SHAPE, "%s: pools must be 16-byte aligned", fn);
  if (cache->dtype == PA_FP8_E4M3 &&
      !(cache->k_scale > 0.f && cache->v_scale > 0.f && std::isfinite(cache->k_scale) &&
        std::isfinite(cache->v_scale)))
    return fail(PA_ERR_SHAPE, "%s: an 8-bit cache needs positive finite k_scale and v_scale", fn);
  if (cache->k_scales != nullptr || cache->v_scales != nullptr) {
    if (cache->dtype != PA_FP8_E4M3)
      return fail(PA_ERR_SHAPE, "%s: per-head scales belong to an 8-bit cache only", fn);
    if (cache->k_scales == nullptr || cache->v_scales == nullptr)
      return fail(PA_ERR_NULL, "%s: k_scales and v_scales go together", fn);
    if ((reinterpret_cast<uintptr_t>(cache->k_scales) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(cache->v_scales) & 3u) != 0)
      return fail(PA_ERR_SHAPE, "%s: k_scales and v_scales must be 4-byte aligned", fn);
  }
  return PA_OK;
}

int check_device_memory(const char* fn, std::initializer_list<NamedPtr> ptrs) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_ERR_SHAPE, "%s: no HIP device is current", fn);
  }
  for (const NamedPtr& np : ptrs) {
    if (np.ptr == nullptr) continue;
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, np.ptr) != hipSuccess) {
      (void)hipGetLastError();
      return fail(PA_ERR_SHAPE, "%s: %s is not memory the HIP runtime knows (a host pointer?)",
                  fn, np.name);
    }
    const bool managed = attr.type == hipMemoryTypeManaged || attr.isManaged != 0;
    if (!managed && !(attr.type == hipMemoryTypeDevice && attr.device == dev))
      return fail(PA_ERR_SHAPE, "%s: %s is not device memory of the current device", fn,
                  np.name);
  }
  return PA_OK;
}

}  // namespace pa

PA_API int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

PA_API int32_t pa_hip_runtime_version(void) {
  int v = 0;
  if (hipRuntimeGetVersion(&v) != hipSuccess) return -1;
  return v;
}

PA_API const char* pa_last_error(void) { return pa::g_error; }

PA_API size_t pa_partials_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                int32_t max_parts) {
  if (num_seqs < 0 || num_heads < 0 || head_dim < 0 || max_parts < 0) return 0;
  const double rows = double(num_seqs) * num_heads * max_parts;
  const double bytes = rows * (double(head_dim) + 2.0) * sizeof(float);
  if (bytes > 9.0e18) return 0;
  return size_t(rows) * (size_t(head_dim) + 2) * sizeof(float);
}
