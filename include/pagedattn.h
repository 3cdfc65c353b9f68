/*
 * pagedattn.h - C ABI of libpagedattn: paged attention decode on AMD Instinct
 * MI355X (gfx950).
 *
 * The KV cache is cut into fixed-size physical blocks; each sequence reaches
 * its blocks through a block table, and attention gathers K/V through that
 * indirection ("How Paged Attention and Continuous Batching Actually Work",
 * section "Paged attention: virtual memory for the KV cache"; "Paged Attention
 * as a Memory Manager", section "How the Kernel Executes Paged Attention").
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - Pointers marked DEVICE are HIP device pointers; HOST pointers are read
 *   before the call returns.  The caller allocates and frees every buffer;
 *   the device entry points below allocate nothing and keep no state besides
 *   a per-thread error message.  (The block manager of pa_block_manager.h
 *   owns host memory for its own state between its create and destroy calls.)
 * - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *   enqueues work on it and returns without synchronising; results are
 *   visible after the stream is synchronised.
 * - Every entry point returns a pa_status.  Argument errors are found on the
 *   host before anything is enqueued (nothing is written then); a failed
 *   launch returns PA_ERR_LAUNCH.  pa_last_error() describes the last
 *   non-OK status of the calling thread.
 * - Pools: two separate buffers, K and V, each laid out
 *   [num_blocks][num_kv_heads][block_size][head_dim] row-major, so the rows of
 *   one (block, KV head) pair are one contiguous run.  Token slot s of the
 *   cache is row (s / block_size, :, s % block_size, :).
 * - Element types: PA_F32 (IEEE binary32), PA_BF16 (bfloat16), or
 *   PA_FP8_E4M3 for an 8-bit cache.  Decode accumulates in binary32 and rounds
 *   a bf16 output to nearest-even.
 * - An 8-bit cache halves the bytes of every block (the lever the
 *   "PagedAttention" glossary page, section "What paging costs", names on top
 *   of paging).  Its codes are OCP E4M3 (1 sign, 4 exponent bits with bias 7,
 *   3 mantissa bits; exponent field 0 = subnormals m/8 * 2^-6; S.1111.111 =
 *   NaN; largest magnitude 448).  Code c of the K pool stands for
 *   e4m3(c) * k_scale, of the V pool for e4m3(c) * v_scale.  Queries and new
 *   tokens of an 8-bit cache are bfloat16.
 * - Device-side contents are not validated beyond what keeps every access in
 *   bounds: a block id outside [0, num_blocks) in a pair, or a slot outside
 *   [0, num_blocks*block_size), is skipped; such a block id in a table is
 *   skipped by the decode entry points (its rows take no part in the softmax)
 *   and read by pa_prefill as zero rows (keys and values of zero); context
 *   lengths are clamped to max_blocks_per_seq*block_size.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 8

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* sizes are negative, inconsistent, or misaligned */
  PA_ERR_UNSUPPORTED = 3, /* a valid request this build has no kernel for */
  PA_ERR_WORKSPACE = 4,   /* workspace or split-KV partial buffers missing or too small */
  PA_ERR_LAUNCH = 5,      /* the HIP runtime refused a launch */
  PA_ERR_ID = 6,          /* unknown request id, or an id already in use (block manager) */
  PA_ERR_STATE = 7,       /* the request's state does not allow the call (block manager) */
  PA_ERR_NOMEM = 8        /* host memory for the block manager could not be allocated */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

/* Description of the two KV pools (a HOST struct holding DEVICE pointers). */
typedef struct pa_cache {
  void *k_pool;          /* DEVICE [num_blocks][num_kv_heads][block_size][head_dim] */
  void *v_pool;          /* DEVICE, same shape and type as k_pool */
  int64_t num_blocks;    /* physical blocks in each pool, > 0 */
  int32_t num_kv_heads;  /* > 0 */
  int32_t block_size;    /* tokens per block: 8, 16 or 32 */
  int32_t head_dim;      /* 64 or 128 */
  int32_t dtype;         /* pa_dtype of both pools */
  float k_scale;         /* PA_FP8_E4M3: dequantisation scales of the pools, positive */
  float v_scale;         /*   and finite; ignored for the other types */
  /* PA_FP8_E4M3 only, optional: one scale per KV head, DEVICE float
   * [num_kv_heads] each, positive and finite, 4-byte aligned; both or
   * neither.  When given they replace k_scale / v_scale: head g's codes are
   * its values divided by k_scales[g] (v_scales[g]).  NULL for the other
   * types. */
  const float *k_scales;
  const float *v_scales;
} pa_cache;

/* Version of this header the library was built from (PA_ABI_VERSION). */
int32_t pa_abi_version(void);

/* Runtime version reported by the HIP runtime the library is bound to
 * (hipRuntimeGetVersion), or -1 if it cannot be queried. */
int32_t pa_hip_runtime_version(void);

/* Message for the calling thread's last non-OK status (HOST string owned by
 * the library, valid until the thread's next failing call); "" if none. */
const char *pa_last_error(void);

/*
 * pa_kv_append - write each new token's K and V rows into the cache.
 *
 * The forward pass writes the new token's K/V through the slot mapping
 * ("How Paged Attention and Continuous Batching Actually Work", section "One
 * step, end to end"; "LLM paged attention arch", section "The architecture:
 * every piece explained").  For token n with s = slot_mapping[n] >= 0, every
 * KV head h gets
 *     K[s / B][h][s % B][:] = k_new[n][h][:],   V likewise from v_new,
 * copied bit for bit (no conversion).  A negative slot means "no write".
 * No other byte of either pool changes.  An 8-bit cache stores instead, for
 * each bf16 input x, the E4M3 code nearest to x / scale (x widened to
 * binary32, the division done in binary32 and rounded to nearest), ties to
 * the even code, magnitudes past 448 clamped to 448, NaN kept as NaN.
 *
 *   cache         HOST   pool description
 *   k_new, v_new  DEVICE [num_tokens][num_kv_heads][head_dim], cache->dtype
 *                        (bfloat16 for an 8-bit cache)
 *   slot_mapping  DEVICE int64 [num_tokens]; live slots must be distinct
 *   num_tokens    >= 0 (0 enqueues nothing)
 * Requires head_dim * element size to be a multiple of 16 bytes and every
 * pointer 16-byte aligned.
 */
int pa_kv_append(const pa_cache *cache, const void *k_new, const void *v_new,
                 const int64_t *slot_mapping, int32_t num_tokens, void *stream);

/*
 * pa_copy_blocks - the copy step of copy-on-write.
 *
 * When a sequence writes into a block it shares, the runtime takes a fresh
 * block and copies the shared content into it ("Paged Attention as a Memory
 * Manager", section "Prefix Caching and Copy-on-Write").  For each pair
 * (src, dst) = (block_pairs[2p], block_pairs[2p+1]) every KV head and row of
 * block src is copied to block dst, in both pools, bit for bit.  Reference
 * counts and table updates belong to the caller's block manager.
 *
 *   block_pairs  DEVICE int64 [num_pairs][2]; destinations distinct and never
 *                also a source (the copies then do not depend on order)
 *   num_pairs    >= 0
 */
int pa_copy_blocks(const pa_cache *cache, const int64_t *block_pairs, int32_t num_pairs,
                   void *stream);

/*
 * pa_swap_blocks - whole-block copies between the device pools and pinned host
 * pools: the data movement of swapping.
 *
 * When the block pool runs dry, a preempted request's KV can be copied to
 * pinned CPU memory and copied back when blocks free up ("LLM paged attention
 * arch", section "The architecture: every piece explained").  For each pair
 * (a, b) = (block_pairs[2p], block_pairs[2p+1]):
 *   PA_SWAP_OUT:  host block b  <- device block a   (K and V pools)
 *   PA_SWAP_IN:   device block b <- host block a
 * every KV head and row, bit for bit.  Pairs whose ids fall outside their pool
 * are skipped.
 *
 *   cache            HOST   the device pools
 *   host_k_pool,     HOST   pinned host memory (hipHostMalloc, or a pinned torch
 *   host_v_pool             tensor) laid out like the device pools, with
 *                           host_num_blocks blocks of the same type; 16-byte aligned
 *   block_pairs      DEVICE int64 [num_pairs][2]; destinations distinct
 *   direction        PA_SWAP_OUT or PA_SWAP_IN
 * Host pools the HIP runtime does not know as pinned memory mapped for the
 * device are refused (PA_ERR_SHAPE) before anything is enqueued.
 */
enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 };

int pa_swap_blocks(const pa_cache *cache, void *host_k_pool, void *host_v_pool,
                   int64_t host_num_blocks, const int64_t *block_pairs, int32_t num_pairs,
                   int32_t direction, void *stream);

/*
 * Attention variants.  The pages name sliding windows and ALiBi as variants a
 * paged kernel has to re-derive its block traversal for ("Paged Attention as
 * a Memory Manager", section "When It Falls Down"); their definitions are the
 * published ones:
 *   sliding_window = W > 0: a query at position p attends to p-W+1 .. p only
 *                    (itself and the W-1 tokens before it); 0: no window.
 *   alibi_slopes:    DEVICE float [num_heads] or NULL; score(t) gains
 *                    slope[h] * (t - p) (Press, Smith and Lewis, "Train Short,
 *                    Test Long: Attention with Linear Biases").
 */
typedef struct pa_attn_variant {
  int32_t sliding_window;
  int32_t reserved;             /* 0 */
  const float *alibi_slopes;
} pa_attn_variant;

/*
 * pa_decode - attention of one query token per sequence over its paged cache.
 *
 * For sequence i, query head h and its KV head g = h / (num_heads/num_kv_heads):
 *     s_t = scale * q[i][h] . K_t      for t < L_i = context_lens[i]
 *     out[i][h] = sum_t softmax(s)_t * V_t
 * with K_t, V_t the rows of logical token t, found through block_tables[i]
 * ("Paged Attention as a Memory Manager", section "How the Kernel Executes
 * Paged Attention": one table read per block, keys loaded per block, scores
 * q.k/sqrt(d_k), padding masked, softmax-weighted value sum; "PagedAttention
 * and continuous batching", section "Attention kernel modification": blocks
 * accumulated with a running softmax).  L_i includes the token appended this
 * step.  Rows at positions >= L_i (or before a sliding window) never affect
 * the result, whatever they hold; L_i = 0 gives a zero output.
 *
 * With a workspace, the (sequence, block) pairs of the whole batch are split
 * evenly over a fixed grid of workgroups, so long and short sequences finish
 * together; the parts of a sequence split between workgroups are merged with
 * the log-sum-exp rule by a second kernel enqueued on the same stream.
 * Without one (workspace = NULL), one workgroup walks each sequence.  The
 * split holds every sequence's first unit in LDS, which bounds it to 16,000
 * sequences: larger batches are walked one workgroup per sequence even with
 * a workspace (the same attention, in the single pass's order and time).
 *
 *   q             DEVICE [num_seqs][num_heads][head_dim], cache->dtype (bfloat16
 *                 for an 8-bit cache, whose K/V values are codes times scales)
 *   block_tables  DEVICE int32 [num_seqs][max_blocks_per_seq]; entries past
 *                 ceil(L_i / block_size) are not read
 *   context_lens  DEVICE int32 [num_seqs], 0 <= L_i <= max_blocks_per_seq*block_size
 *   num_heads     multiple of num_kv_heads; ratio G = 1..8, or 16 for a bf16 or
 *                 8-bit cache (other ratios: PA_ERR_UNSUPPORTED)
 *   scale         > 0 and finite (normally 1/sqrt(head_dim))
 *   variant       HOST pa_attn_variant, or NULL for plain attention.  The query
 *                 sits at position p = L_i - 1: a window W keeps t >= L_i - W
 *                 (blocks wholly before it are neither read nor counted in the
 *                 split), and ALiBi adds slope[h] * (t - p) to s_t.
 *                 sliding_window < 0 or misaligned slopes give PA_ERR_SHAPE.
 *   out           DEVICE [num_seqs][num_heads][head_dim] of out_dtype, 16-byte aligned
 *   out_dtype     PA_F32, or PA_BF16 for a bf16 or 8-bit cache
 *   workspace     DEVICE scratch of workspace_bytes >= pa_decode_workspace_bytes(),
 *                 256-byte aligned, or NULL; its contents need no initialising
 *                 and are meaningless afterwards.  Calls in flight at the same
 *                 time must not share one.
 */
int pa_decode(const pa_cache *cache, const void *q, const int32_t *block_tables,
              const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
              int32_t max_blocks_per_seq, float scale, const pa_attn_variant *variant,
              void *out, int32_t out_dtype, void *workspace, size_t workspace_bytes,
              void *stream);

/*
 * pa_decode_static - pa_decode with the balanced split, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).
 *
 * The same computation, kernels and results, bit for bit, as pa_decode with
 * a workspace; the workspace is instead a 32 MiB array inside the library,
 * one per device, allocated when the library's device code is loaded and
 * held until the process ends.  The call allocates and frees nothing.  All
 * calls on one device share that array: calls that overlap in time on one
 * device (other streams, other host threads) race and give wrong results;
 * calls on different devices do not.  Nothing in the array needs to start at
 * any value.  Sizes whose split needs more than 32 MiB (roughly
 * (1,024 + num_seqs) * num_heads rows of head_dim + 2 floats on a 256-CU
 * device) return PA_ERR_WORKSPACE; more than 16,000 sequences take the
 * single-pass walk, which needs no scratch.  Other arguments and errors are
 * those of pa_decode.
 */
int pa_decode_static(const pa_cache *cache, const void *q, const int32_t *block_tables,
                     const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                     int32_t max_blocks_per_seq, float scale, const pa_attn_variant *variant,
                     void *out, int32_t out_dtype, void *stream);

/*
 * pa_decode_append - one decode step in one launch: the append of every
 * sequence's new token, then pa_decode.
 *
 * Sequence i's token sits at position p = L_i - 1 ("How Paged Attention and
 * Continuous Batching Actually Work", section "One step, end to end": the
 * forward pass writes the token's K/V through the slot mapping, then attention
 * reads the cache); its slot is block_tables[i][p / block_size] * block_size +
 * p % block_size.  The result - pools and out - equals pa_kv_append with
 * those slots followed by pa_decode with the same arguments, bit for bit.  The
 * wave that writes a row is the one that reads it back later in the launch,
 * so no other ordering is needed.  Sequences with L_i = 0, or whose last table
 * entry is outside the pool, write nothing.
 *
 *   k_new, v_new  DEVICE [num_seqs][num_kv_heads][head_dim], the cache type
 *                 (bfloat16 for an 8-bit cache, quantised with the cache's
 *                 scales as pa_kv_append does), 16-byte aligned
 * All other arguments, the workspace and the errors are those of pa_decode.
 */
int pa_decode_append(const pa_cache *cache, const void *q, const void *k_new, const void *v_new,
                     const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
                     int32_t num_heads, int32_t max_blocks_per_seq, float scale,
                     const pa_attn_variant *variant, void *out, int32_t out_dtype,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes pa_decode needs on the current device for these sizes,
 * whatever the pools (0 for a negative or zero size): a bound over every
 * element type, block size and KV-head count.  pa_decode_workspace_size gives
 * the exact need for given pools. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim);

/* Workspace bytes pa_decode (and pa_decode_append) need on the current device
 * for this cache and these sizes; 0 for sizes pa_decode refuses.  The
 * workspace holds the split description and one partial row per (workgroup
 * + sequence, query head) for the parts of split sequences. */
size_t pa_decode_workspace_size(const pa_cache *cache, int32_t num_seqs, int32_t num_heads);

/*
 * pa_prefill - causal attention of a mixed batch: many query tokens per
 * sequence (prompt slices) and single tokens (decodes) in one call.
 *
 * Every scheduled token of the batch is flattened into one sequence of query
 * rows; metadata says where each request's tokens begin and end and what they
 * may see ("How Paged Attention and Continuous Batching Actually Work",
 * section "Continuous batching: schedule steps, not batches").  Sequence i owns
 * rows query_start[i] .. query_start[i+1]-1 of q; its n_i tokens are its last
 * n_i positions, so token j sits at position p = context_lens[i] - n_i + j,
 * and it attends causally to positions 0..p, whose K/V rows are gathered block
 * by block through block_tables[i] ("PagedAttention and continuous batching",
 * section "Attention kernel modification"):
 *     out[row][h] = sum_{t <= p} softmax_t(scale * q[row][h] . K_t) V_t
 * The K/V of all of a sequence's context_lens[i] positions (this step's tokens
 * included, written by pa_kv_append) must be in the cache.  For a bf16 output
 * the softmax weights are rounded to bf16 for the matrix product (round to
 * nearest even, each within 2^-8 of its value, relative) and normalised by the
 * sum of the rounded weights; for a float32 output each weight enters the
 * product as three bf16 terms (within 2^-24 of it) and is normalised by the
 * sum of the float32 weights (three times the P.V matrix work).
 *
 *   q             DEVICE [num_tokens][num_heads][128] bfloat16
 *   block_tables  DEVICE int32 [num_seqs][max_blocks_per_seq]
 *   query_start   DEVICE int32 [num_seqs + 1], rising from 0 to num_tokens
 *   context_lens  DEVICE int32 [num_seqs], n_i <= L_i <= max_blocks_per_seq*block_size
 *                 (rows before position 0, n_i > L_i, get zeros)
 *   num_heads     ratio G to num_kv_heads 1..8 or 16 (a workgroup tile holds
 *                 floor(128 / G) tokens)
 *   out           DEVICE [num_tokens][num_heads][128] of out_dtype (PA_F32 or PA_BF16),
 *                 16-byte aligned; rows of sequences with n_i = 0 are not written
 *   variant       HOST pa_attn_variant, or NULL for plain causal attention
 *   workspace     DEVICE scratch, >= pa_prefill_workspace_bytes(), 256-byte aligned;
 *                 contents need no initialising.  Calls in flight at the same time
 *                 must not share one.
 * Supported: bf16 and 8-bit (E4M3) caches, head_dim 128, block_size 8, 16 or 32.
 * Decode rows (n_i = 1) are computed like the others, with or without a variant.
 */
int pa_prefill(const pa_cache *cache, const void *q, const int32_t *block_tables,
               const int32_t *query_start, const int32_t *context_lens, int32_t num_seqs,
               int32_t num_tokens, int32_t num_heads, int32_t max_blocks_per_seq, float scale,
               const pa_attn_variant *variant, void *out, int32_t out_dtype, void *workspace,
               size_t workspace_bytes, void *stream);

/* Workspace bytes pa_prefill needs for these sizes (0 for invalid sizes). */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                  int32_t num_kv_heads);

/*
 * pa_decode_partitions - split-KV decode: per-partition partial results.
 *
 * Same attention as pa_decode, cut along each sequence's context into
 * partitions of partition_size tokens (a multiple of block_size): partition p
 * of sequence i covers positions [p*P, min((p+1)*P, L_i)).  For p < ceil(L_i/P)
 * it writes, for every query head h,
 *     part_out[i][h][p][:] = the partition's softmax-weighted V sum,
 *     part_max[i][h][p]    = its largest score s_t (natural units),
 *     part_sum[i][h][p]    = sum over it of exp(s_t - part_max),
 * and nothing else; pa_splitkv_reduce merges them.  Requires
 * L_i <= max_parts * P; later partitions are not computed.
 *
 *   part_out      DEVICE float [num_seqs][num_heads][max_parts][head_dim], 16-byte aligned
 *   part_max, part_sum  DEVICE float [num_seqs][num_heads][max_parts]
 *   max_parts     in [1, 65535]
 */
int pa_decode_partitions(const pa_cache *cache, const void *q, const int32_t *block_tables,
                         const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                         int32_t max_blocks_per_seq, float scale, int32_t partition_size,
                         float *part_out, float *part_max, float *part_sum, int32_t max_parts,
                         void *stream);

/*
 * pa_splitkv_reduce - merge split-KV partials with their log-sum-exp weights.
 *
 * Not described on the pages, which run one softmax over the whole context;
 * this is the exact regrouping of that softmax over partitions.  For each
 * (i, h), over the ceil(L_i / partition_size) partitions of sequence i:
 *     M   = max_p part_max[p];   w_p = part_sum[p] * exp(part_max[p] - M)
 *     out = sum_p w_p * part_out[p] / sum_p w_p
 *     lse = M + ln(sum_p w_p)
 * Partitions past a sequence's last are not read.  L_i = 0 gives out = 0 and
 * lse = -inf.
 *
 * Partitions whose part_sum is 0 take no part (their rows are not used).
 *
 *   part_out, part_max, part_sum  DEVICE, as written by pa_decode_partitions;
 *                 part_out 16-byte aligned
 *   context_lens  DEVICE int32 [num_seqs], the same lengths pa_decode_partitions saw
 *   out           DEVICE [num_seqs][num_heads][head_dim] of out_dtype, 16-byte aligned
 *   lse           DEVICE float [num_seqs][num_heads], or NULL
 * Misaligned part_out or out give PA_ERR_SHAPE.
 */
int pa_splitkv_reduce(const float *part_out, const float *part_max, const float *part_sum,
                      const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                      int32_t head_dim, int32_t max_parts, int32_t partition_size, void *out,
                      int32_t out_dtype, float *lse, void *stream);

/* Bytes of part_out + part_max + part_sum for the given sizes (0 on overflow
 * or a negative size). */
size_t pa_partials_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                         int32_t max_parts);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
