// pa_splitkv_reduce: merge split-KV partials with log-sum-exp weights.
//
// One wave per (sequence, query head).  Lane p computes the weight of
// partition p (64 partitions per pass), the wave reduces the maximum and the
// weight sum across lanes, and every lane accumulates D/64 output dims over
// the partitions, reading each partition's output row with coalesced loads.
#include "pa_decode_kernel.h"
#include "pa_internal.h"

namespace pa {
namespace {

struct ReduceArgs {
  const float* part_out;
  const float* part_max;
  const float* part_sum;
  const int32_t* context_lens;
  void* out;
  float* lse;
  int32_t num_heads;
  int32_t max_parts;
  int32_t partition_size;
  int32_t out_f32;
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

template <int D>
__global__ void __launch_bounds__(64) reduce_kernel(ReduceArgs a) {
  constexpr int PER = D / 64;
  constexpr float NEG_INF = -__builtin_inff();
  const int lane = threadIdx.x;
  const int head = blockIdx.x;
  const int seq = blockIdx.y;
  const size_t row = size_t(seq) * a.num_heads + head;
  int len = a.context_lens[seq];
  len = len < 0 ? 0 : len;
  int nparts = int((int64_t(len) + a.partition_size - 1) / a.partition_size);
  nparts = nparts > a.max_parts ? a.max_parts : nparts;
  const size_t base = row * a.max_parts;

  float big = NEG_INF;
  for (int p = lane; p < nparts; p += 64) {
    if (a.part_sum[base + p] > 0.f) big = fmaxf(big, a.part_max[base + p]);
  }
  big = wave_max(big);

  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (big != NEG_INF) {
    for (int p0 = 0; p0 < nparts; p0 += 64) {
      const int p = p0 + lane;
      float w = 0.f;
      if (p < nparts) {
        const float s = a.part_sum[base + p];
        w = s > 0.f ? s * __expf(a.part_max[base + p] - big) : 0.f;
      }
      wsum += w;
      const int cnt = nparts - p0 < 64 ? nparts - p0 : 64;
      const float* rows = a.part_out + (base + p0) * D + lane;
      for (int j = 0; j < cnt; ++j) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
        if (wj == 0.f) continue;  // uniform: skips empty partitions without reading them
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj, rows[size_t(j) * D + e * 64], acc[e]);
      }
    }
  }
  wsum = wave_sum(wsum);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float val = acc[e] * inv;
    const size_t idx = row * D + e * 64 + lane;
    if (a.out_f32)
      static_cast<float*>(a.out)[idx] = val;
    else
      static_cast<uint16_t*>(a.out)[idx] = dev::to_bf16(val);
  }
  if (a.lse && lane == 0) a.lse[row] = wsum > 0.f ? big + __logf(wsum) : NEG_INF;
}

}  // namespace
}  // namespace pa

PA_API int pa_splitkv_reduce(const float* part_out, const float* part_max, const float* part_sum,
                             const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                             int32_t head_dim, int32_t max_parts, int32_t partition_size,
                             void* out, int32_t out_dtype, float* lse, void* stream) {
  using namespace pa;
  const char* fn = "pa_splitkv_reduce";
  if (num_seqs < 0 || num_heads <= 0 || max_parts <= 0 || partition_size <= 0)
    return fail(PA_ERR_SHAPE,
                "%s: need num_seqs >= 0 and positive num_heads, max_parts, partition_size", fn);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128 (got %d)", fn, head_dim);
  if (out_dtype != PA_F32 && out_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: unknown out_dtype %d", fn, out_dtype);
  if (num_seqs > 65535 || num_heads > 65535)
    return fail(PA_ERR_UNSUPPORTED, "%s: at most 65535 sequences and heads", fn);
  if (num_seqs == 0) return PA_OK;
  if (!part_out || !part_max || !part_sum)
    return fail(PA_ERR_WORKSPACE, "%s: part_out, part_max or part_sum is NULL", fn);
  if (!context_lens || !out) return fail(PA_ERR_NULL, "%s: context_lens or out is NULL", fn);
  if (int st = check_device_memory(fn, {{"part_out", part_out}, {"part_max", part_max},
                                        {"part_sum", part_sum}, {"context_lens", context_lens},
                                        {"out", out}, {"lse", lse}}))
    return st;
  ReduceArgs a;
  a.part_out = part_out;
  a.part_max = part_max;
  a.part_sum = part_sum;
  a.context_lens = context_lens;
  a.out = out;
  a.lse = lse;
  a.num_heads = num_heads;
  a.max_parts = max_parts;
  a.partition_size = partition_size;
  a.out_f32 = out_dtype == PA_F32 ? 1 : 0;
  const dim3 grid(static_cast<unsigned>(num_heads), static_cast<unsigned>(num_seqs));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 64)
    hipLaunchKernelGGL(reduce_kernel<64>, grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(reduce_kernel<128>, grid, dim3(64), 0, s, a);
  return launch_result(fn);
}
