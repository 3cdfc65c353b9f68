// pa_decode: host-side validation and dispatch of the decode kernel.
#include <cmath>

#include "pa_decode_kernel.h"
#include "pa_internal.h"

PA_API int pa_decode(const pa_cache* cache, const void* q, const int32_t* block_tables,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                     int32_t max_blocks_per_seq, float scale, int32_t partition_size, void* out,
                     int32_t out_dtype, float* part_out, float* part_max, float* part_sum,
                     int32_t max_parts, void* stream) {
  using namespace pa;
  const char* fn = "pa_decode";
  if (int st = check_cache(cache, fn)) return st;
  if (num_seqs < 0 || num_heads <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_SHAPE, "%s: need num_seqs >= 0, num_heads > 0, max_blocks_per_seq > 0",
                fn);
  if (num_heads % cache->num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "%s: num_heads (%d) is not a multiple of num_kv_heads (%d)", fn,
                num_heads, cache->num_kv_heads);
  const int group = num_heads / cache->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PA_ERR_UNSUPPORTED, "%s: query heads per KV head must be 1, 2, 4 or 8 (got %d)",
                fn, group);
  if (cache->head_dim != 64 && cache->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128 (got %d)", fn,
                cache->head_dim);
  if (cache->block_size != 16 && cache->block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size must be 16 or 32 (got %d)", fn,
                cache->block_size);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PA_ERR_SHAPE, "%s: scale must be positive and finite", fn);
  if (num_seqs > 65535 || cache->num_kv_heads > 65535)
    return fail(PA_ERR_UNSUPPORTED, "%s: at most 65535 sequences and KV heads", fn);
  if (int64_t(max_blocks_per_seq) * cache->block_size > INT32_MAX)
    return fail(PA_ERR_SHAPE, "%s: max_blocks_per_seq too large", fn);
  const bool bf16 = cache->dtype == PA_BF16;
  const bool split = partition_size > 0;
  if (partition_size < 0) return fail(PA_ERR_SHAPE, "%s: partition_size < 0", fn);
  if (split) {
    if (partition_size % cache->block_size != 0)
      return fail(PA_ERR_SHAPE, "%s: partition_size must be a multiple of block_size", fn);
    if (max_parts <= 0) return fail(PA_ERR_WORKSPACE, "%s: max_parts must be positive", fn);
    if (!part_out || !part_max || !part_sum)
      return fail(PA_ERR_WORKSPACE, "%s: split-KV needs part_out, part_max and part_sum", fn);
    if (!aligned16(part_out))
      return fail(PA_ERR_SHAPE, "%s: part_out must be 16-byte aligned", fn);
  } else {
    if (!out) return fail(PA_ERR_NULL, "%s: out is NULL", fn);
    if (out_dtype != PA_F32 && out_dtype != cache->dtype)
      return fail(PA_ERR_UNSUPPORTED, "%s: out_dtype must be PA_F32 or the cache dtype", fn);
  }
  if (num_seqs == 0) return PA_OK;
  if (!q || !block_tables || !context_lens)
    return fail(PA_ERR_NULL, "%s: q, block_tables or context_lens is NULL", fn);
  if (!aligned16(q)) return fail(PA_ERR_SHAPE, "%s: q must be 16-byte aligned", fn);

  DecodeArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.k_pool = static_cast<const uint8_t*>(cache->k_pool);
  a.v_pool = static_cast<const uint8_t*>(cache->v_pool);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.part_out = part_out;
  a.part_max = part_max;
  a.part_sum = part_sum;
  a.num_blocks = cache->num_blocks;
  a.num_kv_heads = cache->num_kv_heads;
  a.num_heads = num_heads;
  a.max_blocks = max_blocks_per_seq;
  a.partition_blocks = split ? partition_size / cache->block_size : 0;
  a.max_parts = split ? max_parts : 1;
  a.out_f32 = (!bf16 || out_dtype == PA_F32) ? 1 : 0;
  a.scale_log2 = scale * 1.4426950408889634f;

  const dim3 grid(unsigned(split ? max_parts : 1), unsigned(cache->num_kv_heads),
                  unsigned(num_seqs));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool ok = bf16 ? launch_decode_bf16(cache->head_dim, cache->block_size, group, a, grid, s)
                       : launch_decode_f32(cache->head_dim, cache->block_size, group, a, grid, s);
  if (!ok) return fail(PA_ERR_UNSUPPORTED, "%s: no kernel for this shape", fn);
  return launch_result(fn);
}
