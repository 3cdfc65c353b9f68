// pa_probe_stream_read: a plain streaming read of device memory, the
// bandwidth reference the decode kernels are measured against.  Every lane
// reads 16-byte chunks with non-temporal loads, 8 in flight, workgroups
// taking consecutive 64 KiB slices in a grid-stride loop; each workgroup
// folds what it read into one 16-byte XOR written to `sink`, so the loads
// cannot be dropped.  Workgroups whose XCD (blockIdx.x % 8, the order the
// dispatcher deals workgroups to the eight XCDs) is not in `xcd_mask` read
// nothing, which measures what a subset of XCDs can pull on its own.
#include "pa_internal.h"
#include "pa_probe.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 512;
constexpr int64_t kSlice = 64 * 1024;                 // bytes a workgroup reads per step
constexpr int kPerLane = kSlice / (kProbeThreads * 16);  // 16-byte loads per lane per slice

__global__ void __launch_bounds__(kProbeThreads)
    stream_read_kernel(const u32x4* src, int64_t slices, int32_t xcd_mask, u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  if ((xcd_mask >> (blockIdx.x % 8)) & 1) {
    // this XCD's workgroups split the slices among themselves
    int nx = 0, rank = 0;
    for (int x = 0; x < 8; ++x) {
      if ((xcd_mask >> x) & 1) {
        if (x < int(blockIdx.x % 8)) ++rank;
        ++nx;
      }
    }
    // workgroups past the last whole round of eight read nothing
    const int64_t per_xcd = gridDim.x / 8;
    const int64_t my = int64_t(blockIdx.x / 8) * nx + rank;
    const int64_t stride = per_xcd * nx;
    for (int64_t s = blockIdx.x / 8 < per_xcd ? my : slices; s < slices; s += stride) {
      const u32x4* p = src + s * (kSlice / 16) + threadIdx.x;
      u32x4 v[kPerLane];
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) v[i] = __builtin_nontemporal_load(p + i * kProbeThreads);
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) acc ^= v[i];
    }
  }
  __shared__ u32x4 red[kProbeThreads / 64];
  for (int off = 32; off > 0; off >>= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] ^= unsigned(__shfl_xor(int(acc[e]), off));
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    u32x4 r = red[0];
    for (int w = 1; w < kProbeThreads / 64; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace
}  // namespace pa

PA_API int pa_probe_stream_read(const void* src, size_t bytes, int32_t workgroups,
                                int32_t xcd_mask, void* sink, void* stream) {
  using namespace pa;
  const char* fn = "pa_probe_stream_read";
  if (bytes == 0) return PA_OK;
  if (!src || !sink) return fail(PA_ERR_NULL, "%s: src or sink is NULL", fn);
  if (bytes % kSlice != 0)
    return fail(PA_ERR_SHAPE, "%s: bytes must be a multiple of %lld", fn, (long long)kSlice);
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 15u) != 0)
    return fail(PA_ERR_SHAPE, "%s: src and sink must be 16-byte aligned", fn);
  if (workgroups < 8 || workgroups > 1 << 20)
    return fail(PA_ERR_SHAPE, "%s: workgroups must be in [8, 2^20]", fn);
  if ((xcd_mask & 0xFF) == 0) return fail(PA_ERR_SHAPE, "%s: xcd_mask selects no XCD", fn);
  if (int st = check_device_memory(fn, {{"src", src}, {"sink", sink}})) return st;
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(workgroups)), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     int64_t(bytes / kSlice), xcd_mask & 0xFF, static_cast<u32x4*>(sink));
  return launch_result(fn);
}
