// pa_decode, pa_decode_partitions, pa_decode_workspace_bytes: host-side
// validation, work decomposition and launch of the decode kernels.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "pa_decode_kernel.h"
#include "pa_internal.h"

namespace pa {
namespace {

int elem_type(int32_t dtype) {
  return dtype == PA_BF16 ? kBF16 : dtype == PA_FP8_E4M3 ? kFP8 : kF32;
}

// Largest workgroup (in waves) made of whole KV heads, at most PA_MAX_WAVES.
int waves_per_group(int num_kv_heads) {
  for (int w : {8, 4, 2, 1})
    if (w <= PA_MAX_WAVES && num_kv_heads % w == 0) return w;
  return 1;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus;
}

// Upper bound on the workgroups of the balanced split: 32 waves per CU.
constexpr int kMaxGroupsPerCu = 32;

// Workgroups the balanced split uses: as many as the device holds at once.
int balanced_groups(const pa_cache* cache, int group, int waves, size_t lds) {
  const int d = cache->head_dim, bs = cache->block_size;
  int per_cu = cache->dtype == PA_BF16       ? decode_groups_per_cu_bf16(d, bs, group, waves, lds)
               : cache->dtype == PA_FP8_E4M3 ? decode_groups_per_cu_fp8(d, bs, group, waves, lds)
                                             : decode_groups_per_cu_f32(d, bs, group, waves, lds);
  if (per_cu < 1) per_cu = 1;
  if (per_cu > kMaxGroupsPerCu) per_cu = kMaxGroupsPerCu;
  return device_cus() * per_cu;
}

// The most one-wave workgroups any decode instantiation fits on a CU (its
// smallest LDS), for the workspace bound that does not know the pools;
// queried once.
int max_groups_per_cu() {
  static std::once_flag once;
  static int best = 1;
  std::call_once(once, [] {
    for (int et : {kF32, kBF16, kFP8})
      for (int d : {64, 128})
        for (int bs : {8, 16, 32})
          for (int g : {1, 2, 3, 4, 5, 6, 7, 8, 16}) {
            if (!decode_group_supported(et, d, bs, g)) continue;
            const size_t lds =
                decode_prefix_lds_bytes(1, true) + decode_wave_lds_bytes(et, d, g, bs);
            const int n = et == kBF16  ? decode_groups_per_cu_bf16(d, bs, g, 1, lds)
                          : et == kFP8 ? decode_groups_per_cu_fp8(d, bs, g, 1, lds)
                                       : decode_groups_per_cu_f32(d, bs, g, 1, lds);
            best = std::max(best, n);
          }
    best = std::min(best, kMaxGroupsPerCu);
  });
  return best;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace of the balanced split: the split description (workgroups used,
// units, first unit of every sequence), then the piece partials, one row per
// (workgroup + sequence, query head).
struct WorkspaceLayout {
  size_t info, piece_out, piece_max, piece_sum, total;
};

WorkspaceLayout layout_for(int64_t groups, int64_t num_seqs, int64_t num_heads, int64_t head_dim) {
  WorkspaceLayout w;
  const int64_t rows = (groups + num_seqs) * num_heads;
  w.info = 0;
  w.piece_out = align_up(size_t(num_seqs + 3) * sizeof(int32_t));
  w.piece_max = w.piece_out + align_up(size_t(rows) * head_dim * sizeof(float));
  w.piece_sum = w.piece_max + align_up(size_t(rows) * sizeof(float));
  w.total = w.piece_sum + align_up(size_t(rows) * sizeof(float));
  return w;
}

// Checks shared by pa_decode and pa_decode_partitions; fills the common args.
int prepare(const char* fn, const pa_cache* cache, const void* q, const int32_t* block_tables,
            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
            int32_t max_blocks_per_seq, float scale, DecodeArgs* a, int* group) {
  if (int st = check_cache(cache, fn)) return st;
  if (num_seqs < 0 || num_heads <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_SHAPE, "%s: need num_seqs >= 0, num_heads > 0, max_blocks_per_seq > 0",
                fn);
  if (num_heads % cache->num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "%s: num_heads (%d) is not a multiple of num_kv_heads (%d)", fn,
                num_heads, cache->num_kv_heads);
  *group = num_heads / cache->num_kv_heads;
  if (cache->head_dim != 64 && cache->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128 (got %d)", fn,
                cache->head_dim);
  if (cache->block_size != 8 && cache->block_size != 16 && cache->block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size must be 8, 16 or 32 (got %d)", fn,
                cache->block_size);
  if (!decode_group_supported(elem_type(cache->dtype), cache->head_dim, cache->block_size,
                              *group))
    return fail(PA_ERR_UNSUPPORTED,
                "%s: query heads per KV head must be 1..8, or 16 for a bf16 or 8-bit cache "
                "(got %d)",
                fn, *group);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PA_ERR_SHAPE, "%s: scale must be positive and finite", fn);
  if (num_seqs > 65535 || cache->num_kv_heads > 65535)
    return fail(PA_ERR_UNSUPPORTED, "%s: at most 65535 sequences and KV heads", fn);
  if (int64_t(max_blocks_per_seq) * cache->block_size > INT32_MAX)
    return fail(PA_ERR_SHAPE, "%s: max_blocks_per_seq too large", fn);
  if (num_seqs > 0) {
    if (!q || !block_tables || !context_lens)
      return fail(PA_ERR_NULL, "%s: q, block_tables or context_lens is NULL", fn);
    if (!aligned16(q)) return fail(PA_ERR_SHAPE, "%s: q must be 16-byte aligned", fn);
  }
  *a = DecodeArgs{};
  a->q = static_cast<const uint8_t*>(q);
  a->k_pool = static_cast<const uint8_t*>(cache->k_pool);
  a->v_pool = static_cast<const uint8_t*>(cache->v_pool);
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->num_blocks = cache->num_blocks;
  a->num_seqs = num_seqs;
  a->num_kv_heads = cache->num_kv_heads;
  a->num_heads = num_heads;
  a->max_blocks = max_blocks_per_seq;
  a->out_f32 = 1;
  // an 8-bit cache's K scale multiplies every score, its V scale every output
  const bool fp8 = cache->dtype == PA_FP8_E4M3;
  // (one scale per KV head: applied per head in the kernel instead)
  const bool per_head = fp8 && cache->k_scales != nullptr;
  a->scale_log2 = scale * 1.4426950408889634f * (fp8 && !per_head ? cache->k_scale : 1.f);
  a->v_scale = fp8 && !per_head ? cache->v_scale : 1.f;
  a->k_scales = per_head ? cache->k_scales : nullptr;
  a->v_scales = per_head ? cache->v_scales : nullptr;
  a->window = 0;
  a->alibi = nullptr;
  return PA_OK;
}

int launch(const char* fn, const pa_cache* cache, int group, const DecodeArgs& a, dim3 grid,
           int waves, size_t lds, hipStream_t s) {
  const int d = cache->head_dim, bs = cache->block_size;
  const bool ok =
      cache->dtype == PA_BF16       ? launch_decode_bf16(d, bs, group, a, grid, waves, lds, s)
      : cache->dtype == PA_FP8_E4M3 ? launch_decode_fp8(d, bs, group, a, grid, waves, lds, s)
                                    : launch_decode_f32(d, bs, group, a, grid, waves, lds, s);
  if (!ok) return fail(PA_ERR_UNSUPPORTED, "%s: no kernel for this shape", fn);
  return launch_result(fn);
}

constexpr int kMaxBalancedSeqs = 16000;  // the unit prefix of all sequences lives in LDS

// The scratch of pa_decode_static: the balanced split's workspace in a
// file-scope device array (each device holds its own copy until the process
// ends), for callers that cannot allocate.  Host code uses the address
// hipGetSymbolAddress gives on each device, never the array's name.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, taken once per device
// with that device current; nullptr (with the message set) on failure.
void* scratch_address(const char* fn) {
  static std::mutex lock;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    fail(PA_ERR_LAUNCH, "%s: no usable current HIP device", fn);
    return nullptr;
  }
  std::lock_guard<std::mutex> guard(lock);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      fail(PA_ERR_LAUNCH, "%s: the static scratch has no address on device %d", fn, dev);
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace
}  // namespace pa

PA_API size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim) {
  using namespace pa;
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0) return 0;
  return layout_for(int64_t(device_cus()) * max_groups_per_cu(), num_seqs, num_heads, head_dim)
      .total;
}

PA_API size_t pa_decode_workspace_size(const pa_cache* cache, int32_t num_seqs,
                                       int32_t num_heads) {
  using namespace pa;
  if (!cache || num_seqs < 0 || num_heads <= 0 || cache->num_kv_heads <= 0 ||
      num_heads % cache->num_kv_heads != 0 || cache->head_dim <= 0)
    return 0;
  const int group = num_heads / cache->num_kv_heads;
  const int et = elem_type(cache->dtype);
  if (!decode_group_supported(et, cache->head_dim, cache->block_size, group)) return 0;
  const int waves = waves_per_group(cache->num_kv_heads);
  const size_t lds =
      decode_prefix_lds_bytes(num_seqs, true) +
      size_t(waves) * decode_wave_lds_bytes(et, cache->head_dim, group, cache->block_size);
  return layout_for(balanced_groups(cache, group, waves, lds), num_seqs, num_heads,
                    cache->head_dim)
      .total;
}

namespace pa {
namespace {

// pa_decode, pa_decode_append when k_new / v_new are given, and
// pa_decode_static when static_scratch is set (the workspace is then the
// file-scope scratch array, and `workspace` is ignored).
int decode_call(const char* fn, const pa_cache* cache, const void* q, const void* k_new,
                const void* v_new, const int32_t* block_tables, const int32_t* context_lens,
                int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq, float scale,
                const pa_attn_variant* variant, void* out, int32_t out_dtype, void* workspace,
                size_t workspace_bytes, void* stream, bool static_scratch = false) {
  DecodeArgs a;
  int group = 0;
  if (int st = prepare(fn, cache, q, block_tables, context_lens, num_seqs, num_heads,
                       max_blocks_per_seq, scale, &a, &group))
    return st;
  if (k_new != nullptr || v_new != nullptr) {
    if (num_seqs > 0 && (!k_new || !v_new))
      return fail(PA_ERR_NULL, "%s: k_new or v_new is NULL", fn);
    if (!aligned16(k_new) || !aligned16(v_new))
      return fail(PA_ERR_SHAPE, "%s: k_new and v_new must be 16-byte aligned", fn);
    a.k_new = static_cast<const uint8_t*>(k_new);
    a.v_new = static_cast<const uint8_t*>(v_new);
    a.k_enc = cache->k_scale;
    a.v_enc = cache->v_scale;
  }
  if (variant) {
    if (variant->sliding_window < 0)
      return fail(PA_ERR_SHAPE, "%s: sliding_window must be >= 0", fn);
    if (variant->alibi_slopes && (reinterpret_cast<uintptr_t>(variant->alibi_slopes) & 3u) != 0)
      return fail(PA_ERR_SHAPE, "%s: alibi_slopes must be 4-byte aligned", fn);
    a.window = variant->sliding_window;
    a.alibi = variant->alibi_slopes;
  }
  if (!out) return fail(PA_ERR_NULL, "%s: out is NULL", fn);
  if (out_dtype != PA_F32 && !(out_dtype == PA_BF16 && cache->dtype != PA_F32))
    return fail(PA_ERR_UNSUPPORTED,
                "%s: out_dtype must be PA_F32, or PA_BF16 for a bf16 or 8-bit cache", fn);
  if (!aligned16(out)) return fail(PA_ERR_SHAPE, "%s: out must be 16-byte aligned", fn);
  if (num_seqs == 0) return PA_OK;
  // (after every other check, right before anything is enqueued)
  auto check_memory = [&]() {
    return check_device_memory(
        fn, {{"k_pool", cache->k_pool}, {"v_pool", cache->v_pool}, {"q", q},
             {"block_tables", block_tables}, {"context_lens", context_lens}, {"out", out},
             {"workspace", static_scratch ? nullptr : workspace}, {"k_new", k_new},
             {"v_new", v_new},
             {"alibi_slopes", a.alibi}, {"k_scales", cache->k_scales},
             {"v_scales", cache->v_scales}});
  };
  a.out = out;
  a.out_f32 = out_dtype == PA_F32 ? 1 : 0;
  const int waves = waves_per_group(cache->num_kv_heads);
  const unsigned head_groups = unsigned(cache->num_kv_heads / waves);
  const hipStream_t s = static_cast<hipStream_t>(stream);

  const size_t wave_lds =
      size_t(waves) * decode_wave_lds_bytes(elem_type(cache->dtype), cache->head_dim, group, cache->block_size);
  if (static_scratch) workspace = nullptr;
  if ((workspace == nullptr && !static_scratch) || num_seqs > kMaxBalancedSeqs) {
    a.mode = kModeSingle;
    if (int st = check_memory()) return st;
    return launch(fn, cache, group, a, dim3(unsigned(num_seqs), head_groups), waves, wave_lds, s);
  }
  const size_t lds = decode_prefix_lds_bytes(num_seqs, true) + wave_lds;
  const int groups = balanced_groups(cache, group, waves, lds);
  const WorkspaceLayout w = layout_for(groups, num_seqs, num_heads, cache->head_dim);
  if (static_scratch) {
    if (w.total > kStaticScratchBytes)
      return fail(PA_ERR_WORKSPACE,
                  "%s: these sizes need %zu bytes of scratch, more than the static %zu", fn,
                  w.total, kStaticScratchBytes);
    workspace = scratch_address(fn);
    if (workspace == nullptr) return PA_ERR_LAUNCH;
    workspace_bytes = kStaticScratchBytes;
  }
  if (workspace_bytes < w.total)
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
                workspace_bytes, w.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(PA_ERR_SHAPE, "%s: workspace must be 256-byte aligned", fn);
  if (int st = check_memory()) return st;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.mode = kModeBalanced;
  a.num_groups = groups;
  a.info = reinterpret_cast<int32_t*>(ws + w.info);
  a.part_out = reinterpret_cast<float*>(ws + w.piece_out);
  a.part_max = reinterpret_cast<float*>(ws + w.piece_max);
  a.part_sum = reinterpret_cast<float*>(ws + w.piece_sum);
  if (int st = launch(fn, cache, group, a, dim3(unsigned(groups), head_groups), waves, lds, s))
    return st;
  MergeArgs m;
  m.piece_out = a.part_out;
  m.piece_max = a.part_max;
  m.piece_sum = a.part_sum;
  m.info = a.info;
  m.out = out;
  m.num_heads = num_heads;
  m.out_f32 = a.out_f32;
  const dim3 mgrid(static_cast<unsigned>((num_heads + 3) / 4), static_cast<unsigned>(num_seqs));
  if (cache->head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, mgrid, dim3(256), 0, s, m);
  else
    hipLaunchKernelGGL(merge_kernel<128>, mgrid, dim3(256), 0, s, m);
  return launch_result(fn);
}

}  // namespace
}  // namespace pa

PA_API int pa_decode(const pa_cache* cache, const void* q, const int32_t* block_tables,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                     int32_t max_blocks_per_seq, float scale, const pa_attn_variant* variant,
                     void* out, int32_t out_dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return pa::decode_call("pa_decode", cache, q, nullptr, nullptr, block_tables, context_lens,
                         num_seqs, num_heads, max_blocks_per_seq, scale, variant, out, out_dtype,
                         workspace, workspace_bytes, stream);
}

PA_API int pa_decode_static(const pa_cache* cache, const void* q, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                            int32_t max_blocks_per_seq, float scale,
                            const pa_attn_variant* variant, void* out, int32_t out_dtype,
                            void* stream) {
  return pa::decode_call("pa_decode_static", cache, q, nullptr, nullptr, block_tables,
                         context_lens, num_seqs, num_heads, max_blocks_per_seq, scale, variant,
                         out, out_dtype, nullptr, 0, stream, true);
}

PA_API int pa_decode_append(const pa_cache* cache, const void* q, const void* k_new,
                            const void* v_new, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                            int32_t max_blocks_per_seq, float scale,
                            const pa_attn_variant* variant, void* out, int32_t out_dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (k_new == nullptr || v_new == nullptr))
    return pa::fail(PA_ERR_NULL, "pa_decode_append: k_new or v_new is NULL");
  return pa::decode_call("pa_decode_append", cache, q, k_new, v_new, block_tables, context_lens,
                         num_seqs, num_heads, max_blocks_per_seq, scale, variant, out, out_dtype,
                         workspace, workspace_bytes, stream);
}

PA_API int pa_decode_partitions(const pa_cache* cache, const void* q, const int32_t* block_tables,
                                const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                int32_t max_blocks_per_seq, float scale, int32_t partition_size,
                                float* part_out, float* part_max, float* part_sum,
                                int32_t max_parts, void* stream) {
  using namespace pa;
  const char* fn = "pa_decode_partitions";
  DecodeArgs a;
  int group = 0;
  if (int st = prepare(fn, cache, q, block_tables, context_lens, num_seqs, num_heads,
                       max_blocks_per_seq, scale, &a, &group))
    return st;
  if (partition_size <= 0 || partition_size % cache->block_size != 0)
    return fail(PA_ERR_SHAPE, "%s: partition_size must be a positive multiple of block_size", fn);
  if (max_parts <= 0 || max_parts > 65535)
    return fail(PA_ERR_WORKSPACE, "%s: max_parts must be in [1, 65535]", fn);
  if (!part_out || !part_max || !part_sum)
    return fail(PA_ERR_WORKSPACE, "%s: part_out, part_max and part_sum are required", fn);
  if (!aligned16(part_out)) return fail(PA_ERR_SHAPE, "%s: part_out must be 16-byte aligned", fn);
  if (num_seqs == 0) return PA_OK;
  if (int st = check_device_memory(
          fn, {{"k_pool", cache->k_pool}, {"v_pool", cache->v_pool}, {"q", q},
               {"block_tables", block_tables}, {"context_lens", context_lens},
               {"part_out", part_out}, {"part_max", part_max}, {"part_sum", part_sum},
               {"k_scales", cache->k_scales}, {"v_scales", cache->v_scales}}))
    return st;
  a.mode = kModePartition;
  a.partition_blocks = partition_size / cache->block_size;
  a.max_parts = max_parts;
  a.part_out = part_out;
  a.part_max = part_max;
  a.part_sum = part_sum;
  const int waves = waves_per_group(cache->num_kv_heads);
  const dim3 grid(unsigned(max_parts), unsigned(cache->num_kv_heads / waves), unsigned(num_seqs));
  const size_t lds =
      size_t(waves) * decode_wave_lds_bytes(elem_type(cache->dtype), cache->head_dim, group, cache->block_size);
  return launch(fn, cache, group, a, grid, waves, lds, static_cast<hipStream_t>(stream));
}
