// pa_prefill: validation, the tile map, and the launch of the attention
// kernel (pa_prefill_kernel.h) for the cache type.
#include "pa_prefill_kernel.h"

namespace pa {
namespace pf {
namespace {

// The tile map: tile t of the grid -> (sequence, tile of that sequence),
// longest walk first.  Workgroups start in grid order (and each XCD takes a
// contiguous run of the map, see the kernels' id remap), so with the tiles
// that walk the most key tiles dispatched first the run ends with short ones
// - a longest-processing-time-first order, which keeps the last long walks
// off the end of the launch and mixes walks that stream keys from memory (a
// decode row's, a long context's) with ones that compute on few.  The order
// does not change any output: every tile writes its own rows.
//
// One workgroup of 1024 threads.  It enumerates the tiles twice, 1024
// sequences at a time: it scans their tile counts, and all threads take the
// chunk's tiles together, each finding the sequence of its tile by binary
// search over the chunk's running ends (a thread per sequence would leave a
// long prompt's hundreds of tiles to one thread).  The first pass counts the
// tiles per walk length (kBuckets buckets of equal width up to the longest
// possible walk), the second places each tile after all tiles of longer
// buckets (within a bucket, in the order the threads' slot claims land).
constexpr int kBuckets = 512;

__global__ void __launch_bounds__(1024) prefill_tiles_kernel(const int32_t* qs,
                                                             const int32_t* context_lens,
                                                             int32_t S, int32_t T, int32_t tt,
                                                             int32_t max_len, int32_t window,
                                                             int32_t* tiles, int32_t max_tiles) {
  __shared__ int32_t s_wave[16];
  __shared__ int32_t s_total;
  __shared__ int32_t s_end[1024];  // end (exclusive) of sequence base + j's tiles in the chunk
  __shared__ int32_t s_count[kBuckets];  // tiles per bucket, then the next free slot
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kBuckets; i += 1024) s_count[i] = 0;
  // key tiles the walk of (sequence seq, tile j) takes, as the attention
  // kernels count them, and its bucket (longest walks in bucket 0)
  const int64_t max_walk = (int64_t(max_len) + kKeys - 1) / kKeys;
  auto bucket = [&](int32_t seq, int32_t j) {
    const int32_t a = min(max(qs[seq], 0), T), b = min(max(qs[seq + 1], 0), T);
    const int32_t n = b - a;
    const int32_t L = min(max(context_lens[seq], 0), max_len);
    const int32_t c = L - n;
    const int32_t j0 = j * tt, j1 = min(j0 + tt, n);
    const int32_t kend = c + j1;
    int64_t walk = 0;
    if (kend > 0 && j1 > j0) {
      const int32_t ntiles = (kend + kKeys - 1) / kKeys;
      const int32_t kt0 = window > 0 ? max(0, c + j0 - window + 1) / kKeys : 0;
      walk = max(ntiles - kt0, 0);
    }
    const int64_t q = walk * kBuckets / (max_walk + 1);
    return kBuckets - 1 - int(min<int64_t>(q, kBuckets - 1));
  };
  int32_t running = 0;
  for (int pass = 0; pass < 2; ++pass) {
    running = 0;
    for (int32_t base = 0; base < S; base += 1024) {
      const int32_t i = base + tid;
      int32_t n = 0;
      if (i < S) {
        const int32_t a = min(max(qs[i], 0), T), b = min(max(qs[i + 1], 0), T);
        n = max(b - a, 0);
      }
      const int32_t cnt = (n + tt - 1) / tt;
      const int32_t incl = wave_inclusive_sum(cnt);
      if (lane == 63) s_wave[wave] = incl;
      __syncthreads();
      if (tid == 0) {
        int32_t acc = 0;
        for (int w = 0; w < 16; ++w) {
          const int32_t v = s_wave[w];
          s_wave[w] = acc;
          acc += v;
        }
        s_total = acc;
      }
      __syncthreads();
      s_end[tid] = s_wave[wave] + incl;
      __syncthreads();
      const int32_t total = s_total;
      for (int32_t t = tid; t < total; t += 1024) {
        int lo = 0, hi = 1023;  // first j with s_end[j] > t (s_end[1023] == total > t)
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s_end[mid] > t) hi = mid; else lo = mid + 1;
        }
        const int32_t start = lo > 0 ? s_end[lo - 1] : 0;
        const int32_t seq_cnt = s_end[lo] - start;
        const int32_t seq = base + lo;
        const int32_t j = seq_cnt - 1 - (t - start);  // the sequence's last tile first
        if (running + t >= max_tiles) continue;
        const int k = bucket(seq, j);
        if (pass == 0) {
          atomicAdd(&s_count[k], 1);
        } else {
          const int32_t slot = atomicAdd(&s_count[k], 1);
          if (slot < max_tiles) {
            tiles[1 + 2 * slot] = seq;
            tiles[2 + 2 * slot] = j;
          }
        }
      }
      running += total;
      __syncthreads();
    }
    if (pass == 0) {
      // bucket counts -> first slot of each bucket (exclusive prefix sum)
      static_assert(kBuckets <= 1024, "one bucket per thread");
      const int32_t v = tid < kBuckets ? s_count[tid] : 0;
      const int32_t incl = wave_inclusive_sum(v);
      if (lane == 63) s_wave[wave] = incl;
      __syncthreads();
      if (tid == 0) {
        int32_t acc = 0;
        for (int w = 0; w < 16; ++w) {
          const int32_t x = s_wave[w];
          s_wave[w] = acc;
          acc += x;
        }
      }
      __syncthreads();
      if (tid < kBuckets) s_count[tid] = s_wave[wave] + incl - v;
      __syncthreads();
    }
  }
  if (tid == 0) tiles[0] = min(running, max_tiles);
}

int32_t tokens_per_tile(int32_t group) { return kRows / group; }

int64_t max_tiles_for(int32_t num_seqs, int32_t num_tokens, int32_t group) {
  const int32_t tt = tokens_per_tile(group);
  return (int64_t(num_tokens) + tt - 1) / tt + num_seqs;
}

}  // namespace
}  // namespace pf
}  // namespace pa

PA_API size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                         int32_t num_kv_heads) {
  if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      num_heads % num_kv_heads != 0)
    return 0;
  const int32_t group = num_heads / num_kv_heads;
  if (!pa::pf::prefill_group_supported(group)) return 0;
  return size_t(1 + 2 * pa::pf::max_tiles_for(num_seqs, num_tokens, group)) * sizeof(int32_t);
}

PA_API int pa_prefill(const pa_cache* cache, const void* q, const int32_t* block_tables,
                      const int32_t* query_start, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_tokens, int32_t num_heads, int32_t max_blocks_per_seq,
                      float scale, const pa_attn_variant* variant, void* out,
                      int32_t out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace pa;
  using namespace pa::pf;
  if (int st = check_cache(cache, "pa_prefill")) return st;
  const int32_t window = variant ? variant->sliding_window : 0;
  const float* alibi = variant ? variant->alibi_slopes : nullptr;
  if (window < 0) return fail(PA_ERR_SHAPE, "pa_prefill: sliding_window must be >= 0");
  if (alibi && (reinterpret_cast<uintptr_t>(alibi) & 3u) != 0)
    return fail(PA_ERR_SHAPE, "pa_prefill: alibi_slopes must be 4-byte aligned");
  if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_SHAPE, "pa_prefill: sizes must be non-negative (heads, table width positive)");
  if (cache->dtype != PA_BF16 && cache->dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: bf16 and 8-bit caches only");
  if (cache->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: head_dim 128 only");
  if (cache->block_size != 8 && cache->block_size != 16 && cache->block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: block_size 8, 16 or 32 only");
  if (num_heads % cache->num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "pa_prefill: num_heads must be a multiple of num_kv_heads");
  const int32_t group = num_heads / cache->num_kv_heads;
  if (!prefill_group_supported(group))
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: heads per KV head must be 1..8 or 16");
  if (!(scale > 0.f) || !(scale < 3.4e38f))
    return fail(PA_ERR_SHAPE, "pa_prefill: scale must be positive and finite");
  if (out_dtype != PA_F32 && out_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: out_dtype must be PA_F32 or PA_BF16");
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!q || !block_tables || !query_start || !context_lens || !out)
    return fail(PA_ERR_NULL, "pa_prefill: a required pointer is NULL");
  if (!aligned16(q) || !aligned16(out))
    return fail(PA_ERR_SHAPE, "pa_prefill: q and out must be 16-byte aligned");
  if (int64_t(max_blocks_per_seq) * cache->block_size > INT32_MAX)
    return fail(PA_ERR_SHAPE, "pa_prefill: table width too large");
  const int64_t max_tiles = max_tiles_for(num_seqs, num_tokens, group);
  if (max_tiles > INT32_MAX / 2 - 1)
    return fail(PA_ERR_SHAPE, "pa_prefill: too many tiles");
  const size_t need = pa_prefill_workspace_bytes(num_seqs, num_tokens, num_heads,
                                                 cache->num_kv_heads);
  if (!workspace || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "pa_prefill: workspace of %zu bytes needed", need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(PA_ERR_SHAPE, "pa_prefill: workspace must be 256-byte aligned");
  if (cache->num_kv_heads > 65535)
    return fail(PA_ERR_SHAPE, "pa_prefill: too many KV heads");
  if (int st = check_device_memory(
          "pa_prefill", {{"k_pool", cache->k_pool}, {"v_pool", cache->v_pool}, {"q", q},
                         {"block_tables", block_tables}, {"query_start", query_start},
                         {"context_lens", context_lens}, {"out", out}, {"workspace", workspace},
                         {"alibi_slopes", alibi}, {"k_scales", cache->k_scales},
                         {"v_scales", cache->v_scales}}))
    return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* tiles = static_cast<int32_t*>(workspace);
  hipLaunchKernelGGL(prefill_tiles_kernel, dim3(1), dim3(1024), 0, s, query_start, context_lens,
                     num_seqs, num_tokens, tokens_per_tile(group),
                     int32_t(int64_t(max_blocks_per_seq) * cache->block_size), window, tiles,
                     int32_t(max_tiles));
  if (int st = launch_result("pa_prefill")) return st;

  PrefillArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.k_pool = static_cast<const uint8_t*>(cache->k_pool);
  a.v_pool = static_cast<const uint8_t*>(cache->v_pool);
  a.block_tables = block_tables;
  a.query_start = query_start;
  a.context_lens = context_lens;
  a.tiles = tiles;
  a.out = out;
  a.num_blocks = cache->num_blocks;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_kv_heads = cache->num_kv_heads;
  a.num_heads = num_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_tiles = int32_t(max_tiles);
  const bool fp8 = cache->dtype == PA_FP8_E4M3;
  const bool per_head = fp8 && cache->k_scales != nullptr;
  a.scale_log2 = scale * 1.4426950408889634f * (fp8 && !per_head ? cache->k_scale : 1.0f);
  a.v_scale = fp8 && !per_head ? cache->v_scale : 1.0f;
  a.k_scales = per_head ? cache->k_scales : nullptr;
  a.v_scales = per_head ? cache->v_scales : nullptr;
  a.window = window;
  a.alibi = alibi;
  const dim3 grid(unsigned(max_tiles), unsigned(cache->num_kv_heads));
  const bool f32 = out_dtype == PA_F32;
  return fp8 ? launch_prefill_fp8(a, cache->block_size, group, f32, grid, s)
             : launch_prefill_bf16(a, cache->block_size, group, f32, grid, s);
}
