// KV writes of a decode step: the new-token append through the slot mapping,
// the block copy of copy-on-write, and the block copies of swapping between
// the device pools and pinned host pools.  All are 16-byte data movement:
// every thread writes one 16-byte chunk, consecutive threads write
// consecutive chunks of a block, so each wave reads and writes whole
// contiguous runs.  An 8-bit cache's append reads 32 bytes of bf16 per chunk
// and quantises them.
#include "pa_e4m3.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxGrid = 65536;

struct AppendArgs {
  uint8_t* k_pool;
  uint8_t* v_pool;
  const uint8_t* k_new;
  const uint8_t* v_new;
  const int64_t* slots;
  int64_t num_slots;        // num_blocks * block_size
  int64_t total_chunks;     // num_tokens * 2 * heads * chunks_per_row
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t chunks_per_row;   // head_dim * element bytes / 16
  int32_t quantize;         // 8-bit cache: bf16 inputs stored as E4M3 codes
  float k_scale;
  float v_scale;
  const float* k_scales;    // per KV head, or NULL (then k_scale / v_scale)
  const float* v_scales;
};

// "How Paged Attention and Continuous Batching Actually Work", section "One
// step, end to end": the forward pass writes the new token's K/V through the
// slot mapping.  Slot s is row (s / B, :, s % B, :) of each pool.
__global__ void __launch_bounds__(kThreads) append_kernel(AppendArgs a) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < a.total_chunks;
       idx += stride) {
    const int64_t chunk = idx % a.chunks_per_row;
    int64_t rest = idx / a.chunks_per_row;
    const int64_t head = rest % a.num_kv_heads;
    rest /= a.num_kv_heads;
    const bool is_v = rest & 1;
    const int64_t token = rest >> 1;
    const int64_t slot = a.slots[token];
    if (slot < 0 || slot >= a.num_slots) continue;
    const int64_t block = slot / a.block_size;
    const int64_t row = slot - block * a.block_size;
    const int64_t src_chunk = (token * a.num_kv_heads + head) * a.chunks_per_row + chunk;
    const int64_t dst_chunk =
        ((block * a.num_kv_heads + head) * a.block_size + row) * a.chunks_per_row + chunk;
    uint4* dst = reinterpret_cast<uint4*>(is_v ? a.v_pool : a.k_pool) + dst_chunk;
    const uint4* src = reinterpret_cast<const uint4*>(is_v ? a.v_new : a.k_new);
    if (!a.quantize) {
      *dst = src[src_chunk];
      continue;
    }
    // 16 bf16 inputs (two 16-byte chunks of the input row) -> 16 codes
    const float* per_head = is_v ? a.v_scales : a.k_scales;
    const float scale = per_head ? per_head[head] : (is_v ? a.v_scale : a.k_scale);
    const uint2 lo = codec::quantize_chunk(src[2 * src_chunk], scale);
    const uint2 hi = codec::quantize_chunk(src[2 * src_chunk + 1], scale);
    *dst = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

struct CopyArgs {
  const uint8_t* src_k;
  const uint8_t* src_v;
  uint8_t* dst_k;
  uint8_t* dst_v;
  const int64_t* pairs;
  int64_t src_blocks;        // blocks in the source pools
  int64_t dst_blocks;        // blocks in the destination pools
  int64_t chunks_per_block;  // heads * block_size * head_dim * element bytes / 16
  int64_t total_chunks;      // num_pairs * 2 * chunks_per_block
};

// Whole-block copies, block src of the source pools to block dst of the
// destination pools.  Copy-on-write copies inside the device pools ("Paged
// Attention as a Memory Manager", section "Prefix Caching and Copy-on-Write":
// the fresh block receives a copy of the shared block's content); a swap
// copies between the device pools and pinned host pools ("LLM paged attention
// arch", section "The architecture: every piece explained").
__global__ void __launch_bounds__(kThreads) copy_kernel(CopyArgs a) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < a.total_chunks;
       idx += stride) {
    const int64_t chunk = idx % a.chunks_per_block;
    const int64_t rest = idx / a.chunks_per_block;
    const bool is_v = rest & 1;
    const int64_t pair = rest >> 1;
    const int64_t src = a.pairs[2 * pair];
    const int64_t dst = a.pairs[2 * pair + 1];
    if (src < 0 || src >= a.src_blocks || dst < 0 || dst >= a.dst_blocks) continue;
    const uint4* from = reinterpret_cast<const uint4*>(is_v ? a.src_v : a.src_k);
    uint4* to = reinterpret_cast<uint4*>(is_v ? a.dst_v : a.dst_k);
    to[dst * a.chunks_per_block + chunk] = from[src * a.chunks_per_block + chunk];
  }
}

unsigned grid_for(int64_t total) {
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  return unsigned(blocks < 1 ? 1 : blocks);
}

}  // namespace
}  // namespace pa

PA_API int pa_kv_append(const pa_cache* cache, const void* k_new, const void* v_new,
                        const int64_t* slot_mapping, int32_t num_tokens, void* stream) {
  using namespace pa;
  if (int st = check_cache(cache, "pa_kv_append")) return st;
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "pa_kv_append: num_tokens < 0");
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping)
    return fail(PA_ERR_NULL, "pa_kv_append: k_new, v_new or slot_mapping is NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PA_ERR_SHAPE, "pa_kv_append: k_new/v_new must be 16-byte aligned");
  // (an 8-bit cache's rows are head_dim bytes; check_cache asks for a multiple of 16)
  if ((reinterpret_cast<uintptr_t>(slot_mapping) & 7u) != 0)
    return fail(PA_ERR_SHAPE, "pa_kv_append: slot_mapping must be 8-byte aligned");
  if (int st = check_device_memory("pa_kv_append",
                                   {{"k_pool", cache->k_pool}, {"v_pool", cache->v_pool},
                                    {"k_new", k_new}, {"v_new", v_new},
                                    {"slot_mapping", slot_mapping},
                                    {"k_scales", cache->k_scales}, {"v_scales", cache->v_scales}}))
    return st;
  AppendArgs a;
  a.k_pool = static_cast<uint8_t*>(cache->k_pool);
  a.v_pool = static_cast<uint8_t*>(cache->v_pool);
  a.k_new = static_cast<const uint8_t*>(k_new);
  a.v_new = static_cast<const uint8_t*>(v_new);
  a.slots = slot_mapping;
  a.num_slots = cache->num_blocks * cache->block_size;
  a.num_kv_heads = cache->num_kv_heads;
  a.block_size = cache->block_size;
  a.chunks_per_row = cache->head_dim * element_bytes(cache->dtype) / 16;
  a.quantize = cache->dtype == PA_FP8_E4M3 ? 1 : 0;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.k_scales = cache->k_scales;
  a.v_scales = cache->v_scales;
  a.total_chunks = int64_t(num_tokens) * 2 * cache->num_kv_heads * a.chunks_per_row;
  hipLaunchKernelGGL(append_kernel, dim3(grid_for(a.total_chunks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return launch_result("pa_kv_append");
}

namespace pa {
namespace {

int launch_copy(CopyArgs a, int32_t num_pairs, const pa_cache* cache, hipStream_t stream,
                const char* fn) {
  a.chunks_per_block = int64_t(cache->num_kv_heads) * cache->block_size * cache->head_dim *
                       element_bytes(cache->dtype) / 16;
  a.total_chunks = int64_t(num_pairs) * 2 * a.chunks_per_block;
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(a.total_chunks)), dim3(kThreads), 0, stream, a);
  return launch_result(fn);
}

// Device address of pinned host memory, or nullptr if the HIP runtime does not
// know `host` as pinned memory mapped for the current device.
void* mapped_host(void* host) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type != hipMemoryTypeHost) return nullptr;
  void* dev = nullptr;
  if (hipHostGetDevicePointer(&dev, host, 0) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return dev;
}

}  // namespace
}  // namespace pa

PA_API int pa_copy_blocks(const pa_cache* cache, const int64_t* block_pairs, int32_t num_pairs,
                          void* stream) {
  using namespace pa;
  if (int st = check_cache(cache, "pa_copy_blocks")) return st;
  if (num_pairs < 0) return fail(PA_ERR_SHAPE, "pa_copy_blocks: num_pairs < 0");
  if (num_pairs == 0) return PA_OK;
  if (!block_pairs) return fail(PA_ERR_NULL, "pa_copy_blocks: block_pairs is NULL");
  if ((reinterpret_cast<uintptr_t>(block_pairs) & 7u) != 0)
    return fail(PA_ERR_SHAPE, "pa_copy_blocks: block_pairs must be 8-byte aligned");
  if (int st = check_device_memory("pa_copy_blocks", {{"k_pool", cache->k_pool},
                                                      {"v_pool", cache->v_pool},
                                                      {"block_pairs", block_pairs}}))
    return st;
  CopyArgs a;
  a.src_k = static_cast<const uint8_t*>(cache->k_pool);
  a.src_v = static_cast<const uint8_t*>(cache->v_pool);
  a.dst_k = static_cast<uint8_t*>(cache->k_pool);
  a.dst_v = static_cast<uint8_t*>(cache->v_pool);
  a.pairs = block_pairs;
  a.src_blocks = a.dst_blocks = cache->num_blocks;
  return launch_copy(a, num_pairs, cache, static_cast<hipStream_t>(stream), "pa_copy_blocks");
}

PA_API int pa_swap_blocks(const pa_cache* cache, void* host_k_pool, void* host_v_pool,
                          int64_t host_num_blocks, const int64_t* block_pairs, int32_t num_pairs,
                          int32_t direction, void* stream) {
  using namespace pa;
  if (int st = check_cache(cache, "pa_swap_blocks")) return st;
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return fail(PA_ERR_SHAPE, "pa_swap_blocks: direction must be PA_SWAP_OUT or PA_SWAP_IN");
  if (num_pairs < 0 || host_num_blocks < 0)
    return fail(PA_ERR_SHAPE, "pa_swap_blocks: num_pairs and host_num_blocks must be >= 0");
  if (num_pairs == 0) return PA_OK;
  if (!block_pairs || !host_k_pool || !host_v_pool)
    return fail(PA_ERR_NULL, "pa_swap_blocks: block_pairs or a host pool is NULL");
  if ((reinterpret_cast<uintptr_t>(block_pairs) & 7u) != 0)
    return fail(PA_ERR_SHAPE, "pa_swap_blocks: block_pairs must be 8-byte aligned");
  if (!aligned16(host_k_pool) || !aligned16(host_v_pool))
    return fail(PA_ERR_SHAPE, "pa_swap_blocks: host pools must be 16-byte aligned");
  if (int st = check_device_memory("pa_swap_blocks", {{"k_pool", cache->k_pool},
                                                      {"v_pool", cache->v_pool},
                                                      {"block_pairs", block_pairs}}))
    return st;
  void* hk = mapped_host(host_k_pool);
  void* hv = mapped_host(host_v_pool);
  if (!hk || !hv)
    return fail(PA_ERR_SHAPE, "pa_swap_blocks: host pools must be pinned host memory mapped "
                              "for the device (hipHostMalloc or a pinned tensor)");
  CopyArgs a;
  a.pairs = block_pairs;
  if (direction == PA_SWAP_OUT) {
    a.src_k = static_cast<const uint8_t*>(cache->k_pool);
    a.src_v = static_cast<const uint8_t*>(cache->v_pool);
    a.dst_k = static_cast<uint8_t*>(hk);
    a.dst_v = static_cast<uint8_t*>(hv);
    a.src_blocks = cache->num_blocks;
    a.dst_blocks = host_num_blocks;
  } else {
    a.src_k = static_cast<const uint8_t*>(hk);
    a.src_v = static_cast<const uint8_t*>(hv);
    a.dst_k = static_cast<uint8_t*>(cache->k_pool);
    a.dst_v = static_cast<uint8_t*>(cache->v_pool);
    a.src_blocks = host_num_blocks;
    a.dst_blocks = cache->num_blocks;
  }
  return launch_copy(a, num_pairs, cache, static_cast<hipStream_t>(stream), "pa_swap_blocks");
}
