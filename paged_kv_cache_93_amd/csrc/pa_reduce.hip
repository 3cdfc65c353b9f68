// pa_splitkv_reduce: merge split-KV partials with log-sum-exp weights.
//
// One wave per (sequence, query head), four heads per workgroup.  Lane p
// holds partition p's maximum and sum (64 partitions per pass), so the
// global maximum and the weights come from one load per lane and a wave
// reduction; the partitions' output rows then come in with 16-byte loads,
// D/4 lanes per row, so one load instruction brings 256/D rows, and eight
// instructions are in flight at a time.  Each lane accumulates its 4 dims of
// the rows it loaded, and the lane groups that share dims add up at the end.
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

template <int D>
__global__ void __launch_bounds__(256) reduce_kernel(ReduceArgs a) {
  using namespace dev;
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int LR = D / 4;        // lanes per row
  constexpr int RPI = 64 / LR;     // rows per load instruction
  constexpr int NBATCH = 8;        // load instructions in flight
  constexpr int PB = RPI * NBATCH;  // partitions per batch
  constexpr float NEG_INF = -__builtin_inff();
  const int lane = threadIdx.x & 63;
  const int head = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int seq = blockIdx.y;
  if (head >= a.num_heads) return;
  const int sub = lane / LR;        // which row of an instruction this lane reads
  const int col = (lane % LR) * 4;  // its 4 dims
  const size_t row = size_t(seq) * a.num_heads + head;
  int len = a.context_lens[seq];
  len = len < 0 ? 0 : len;
  int nparts = int((int64_t(len) + a.partition_size - 1) / a.partition_size);
  nparts = nparts > a.max_parts ? a.max_parts : nparts;
  const size_t base = row * a.max_parts;
  const float* rows = a.part_out + base * D + col;

  f4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f, big = NEG_INF;
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    const int cnt = min(64, nparts - p0);
    float pm = NEG_INF, ps = 0.f;
    if (lane < cnt) {
      ps = a.part_sum[base + p0 + lane];
      pm = a.part_max[base + p0 + lane];
    }
    f4 v[NBATCH];
#pragma unroll
    for (int i = 0; i < NBATCH; ++i) {
      const int p = i * RPI + sub;
      v[i] = p < cnt ? *reinterpret_cast<const f4*>(rows + size_t(p0 + p) * D) : f4{0.f, 0.f, 0.f, 0.f};
    }
    // running maximum over partitions with weight, rescaling what came before
    float cmax = ps > 0.f ? pm : NEG_INF;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off));
    const float nb = fmaxf(big, cmax);
    if (nb != big) {
      const float f = big == NEG_INF ? 0.f : __expf(big - nb);
      acc *= f;
      wsum *= f;
      big = nb;
    }
    const float w = ps > 0.f ? ps * __expf(pm - big) : 0.f;
    float ws = w;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) ws += __shfl_xor(ws, off);
    wsum += ws;
    for (int b0 = 0; b0 < cnt; b0 += PB) {
      if (b0 > 0) {
#pragma unroll
        for (int i = 0; i < NBATCH; ++i) {
          const int p = b0 + i * RPI + sub;
          v[i] = p < cnt ? *reinterpret_cast<const f4*>(rows + size_t(p0 + p) * D)
                         : f4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int i = 0; i < NBATCH; ++i) {
        const int p = b0 + i * RPI + sub;  // < 64; lanes past cnt hold w = 0
        const float wp = __shfl(w, p);
        // a partition with no weight is left out (its row may hold anything)
        if (wp != 0.f) acc += wp * v[i];
      }
    }
  }
  // add up the RPI row groups of each load instruction
#pragma unroll
  for (int off = LR; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  if (lane < LR) {
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const size_t o = row * D + col;
    if (a.out_f32) {
      *reinterpret_cast<f4*>(static_cast<float*>(a.out) + o) = acc * inv;
    } else {
      uint16_t* dst = static_cast<uint16_t*>(a.out) + o;
      const uint32_t lo = to_bf16(acc[0] * inv) | (to_bf16(acc[1] * inv) << 16);
      const uint32_t hi = to_bf16(acc[2] * inv) | (to_bf16(acc[3] * inv) << 16);
      *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
    }
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
  if (!aligned16(part_out) || !aligned16(out))
    return fail(PA_ERR_SHAPE, "%s: part_out and out must be 16-byte aligned", fn);
  const dim3 grid(static_cast<unsigned>((num_heads + 3) / 4), static_cast<unsigned>(num_seqs));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 64)
    hipLaunchKernelGGL(reduce_kernel<64>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(reduce_kernel<128>, grid, dim3(256), 0, s, a);
  return launch_result(fn);
}
