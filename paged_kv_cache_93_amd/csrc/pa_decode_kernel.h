// Paged attention decode kernel for gfx950 (wave64).
//
// What it computes ("Paged Attention as a Memory Manager", section "How the
// Kernel Executes Paged Attention"; "PagedAttention and continuous batching",
// section "Attention kernel modification"): for one sequence and one KV head,
// walk the sequence's blocks, read each block's physical id from the block
// table once, load the block's key rows, score them against the G query heads
// that share the KV head (q.k scaled), mask rows past the context length, and
// fold the block into a running softmax of the value rows.
//
// Mapping onto CDNA4 (the pages' warp-of-32 thread groups are not used):
// * A workgroup has one wave per KV head of a head group (up to 8).  All its
//   waves walk the same blocks, so the rows of all heads of a block - one
//   contiguous run in each pool - are read at about the same time.  The waves
//   meet at no barrier after the preamble; each owns its head end to end and
//   only publishes its progress, so that the two waves sharing a SIMD keep
//   pace (the one behind runs at raised issue priority).
// * Work unit = one (sequence, block), or on the MFMA path with 8-token
//   blocks a pair of consecutive blocks (one 16-row tile).  Three ways to
//   hand units out:
//   single pass (a workgroup per sequence), fixed partitions (a workgroup per
//   (sequence, partition), writing split-KV partials), and balanced (a fixed
//   grid; all units of the batch are split evenly over the workgroups, so a
//   workgroup's range holds whole sequences and pieces of sequences; whole
//   ones write the output, pieces write partials merged by merge_kernel).
// * Rows are loaded in 16-byte chunks with non-temporal loads (the cache is
//   streamed once); one load instruction covers 1 KiB of contiguous rows.
// * q.k, bf16 and 8-bit caches with 64- or 128-dim heads (blocks of 8, 16 or 32): a
//   16-row K tile goes through LDS into the MFMA A layout and D/32
//   v_mfma_f32_16x16x32_bf16 score it against the G query heads (the B
//   operand; columns past G are ignored).  P.V then runs on MFMA too: the
//   weights, in lane 16g + h for rows 4g..4g+3 of head h, are already the B
//   operand of O^T += V^T P, and the V tile goes through the same LDS area and
//   comes back transposed (ds_read_b64_tr_b16) as the A operand; each weight
//   enters as three bf16 terms, so the product keeps it to 2^-23.  Float32
//   caches: each lane dots its
//   16-byte chunk against the same chunk of each query head (v_dot2 for bf16
//   pairs, f32 accumulation), the lanes of a row add up their partial sums
//   with DPP row rotations, and the V rows are accumulated on the VALU in f32.
// * Running softmax in log2 units (s*scale*log2 e), so weights are exp2(s - m).
//   On the VALU path row groups (lanes that see the same rows) keep their own
//   running state and are merged once per piece with the log-sum-exp rule; on
//   the MFMA path the four row groups of a head share one base.
// * The workgroup's units are walked as one stream: a ring of PF+1 register
//   tiles keeps the next PF tiles in flight while the current one is scored,
//   across piece boundaries too.  Block-table entries, context lengths and
//   block indices of 64 units at a time are fetched with one vector load per
//   lane (one window ahead) and handed out with v_readlane, so each table
//   entry is read once.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_e4m3.h"

namespace pa {

enum DecodeMode : int32_t { kModeSingle = 0, kModePartition = 1, kModeBalanced = 2 };

// Element type of the K/V pools (the template parameter ET of decode_kernel).
enum ElemType : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

struct DecodeArgs {
  const uint8_t* q;
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;            // final output (single and balanced modes)
  float* part_out;      // partition partials, or balanced-mode pieces
  float* part_max;
  float* part_sum;
  int32_t* info;        // balanced: [0] workgroups used, [1] units, [2 + i] first unit of sequence i
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t num_heads;
  int32_t max_blocks;
  int32_t mode;
  int32_t partition_blocks;  // partition mode: blocks per partition
  int32_t max_parts;         // partition mode: partitions per (sequence, head) row
  int32_t num_groups;        // balanced mode: workgroups in the grid (those past the unit count idle)
  int32_t out_f32;           // 1: binary32 output; 0: bf16 output (bf16 or 8-bit cache)
  float scale_log2;          // score scale * log2(e), times the K pool's scale (8-bit cache)
  float v_scale;             // the V pool's scale (8-bit cache), else 1
  int32_t window;            // sliding window in tokens (0: none): attend to L-W .. L-1
  const float* alibi;        // ALiBi slope per query head, or NULL
  // Fused append (single and balanced modes): sequence i's new-token K and V
  // rows, [num_seqs][num_kv_heads][D] of the cache type (bf16 for an 8-bit
  // cache), written at position L_i - 1 through its block table before they
  // are read; NULL: none.  k_enc / v_enc: an 8-bit cache's pool scales.
  const uint8_t* k_new;
  const uint8_t* v_new;
  float k_enc;
  float v_enc;
  // 8-bit cache with one scale per KV head (or NULL): k_scales[g] multiplies
  // head g's scores (scale_log2 then leaves it out) and also encodes the fused
  // append's K codes; v_scales[g] its outputs and V codes
  const float* k_scales;
  const float* v_scales;
};

namespace dev {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// What one lane loads of a row: 16 bytes, or 8 bytes (eight E4M3 codes).
template <int LB> struct LaneChunk { typedef u32x4 type; };
template <> struct LaneChunk<8> { typedef u32x2 type; };

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994531f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xF, 0xF, true);
}

// Sum over aligned groups of W lanes; every lane of a group gets the same bits
// (each step adds a symmetric pair of partial sums).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W == 8 || W == 16 || W == 32, "group width");
  if constexpr (W == 8) {
    x += dpp<0x141>(x);  // row_half_mirror: lane i <-> 7-i inside 8 lanes
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  } else {
    x += dpp<0x128>(x);  // row_ror:8
    x += dpp<0x124>(x);  // row_ror:4
    x += dpp<0x122>(x);  // row_ror:2
    x += dpp<0x121>(x);  // row_ror:1
    if constexpr (W == 32) x += __shfl_xor(x, 16);
  }
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The values of lanes l and l ^ OFF, lower lane first, in both lanes.  OFF = 16
// and 32 use gfx950's lane swaps (v_permlane16/32_swap: plain VALU, no LDS
// round trip); smaller offsets a shuffle.
template <int OFF>
__device__ __forceinline__ void xor_pair(float x, float& lo, float& hi) {
  const unsigned int u = __float_as_uint(x);
  if constexpr (OFF == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  } else {
    const float o = __shfl_xor(x, OFF);
    const bool upper = (threadIdx.x & OFF) != 0;
    lo = upper ? o : x;
    hi = upper ? x : o;
  }
}

// Sum (or max) over lanes that differ only in bits FROM.. of the lane index
// (FROM a power of two); every lane of a set gets the same bits.
template <int FROM>
__device__ __forceinline__ float xor_sum(float x) {
  if constexpr (FROM >= 64) {
    return x;
  } else {
    float lo, hi;
    xor_pair<FROM>(x, lo, hi);
    return xor_sum<FROM * 2>(lo + hi);
  }
}
template <int FROM>
__device__ __forceinline__ float xor_max(float x) {
  if constexpr (FROM >= 64) {
    return x;
  } else {
    float lo, hi;
    xor_pair<FROM>(x, lo, hi);
    return xor_max<FROM * 2>(fmaxf(lo, hi));
  }
}

// Sum and maximum over the 64 lanes of a wave, the same bits in every lane:
// DPP row rotations inside each row of 16, then the lane swaps across rows.
__device__ __forceinline__ float wave_sum(float x) { return xor_sum<16>(group_sum<16>(x)); }
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0x128>(x));  // row_ror:8
  x = fmaxf(x, dpp<0x124>(x));  // row_ror:4
  x = fmaxf(x, dpp<0x122>(x));  // row_ror:2
  x = fmaxf(x, dpp<0x121>(x));  // row_ror:1
  return xor_max<16>(x);
}

// Inclusive prefix sum over the 64 lanes: shifted adds inside each row of 16
// lanes (DPP row_shr), then the running totals of rows 0 and 0..1 carried
// into the rows after them (DPP row_bcast:15 and row_bcast:31).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

template <bool NT, class T>
__device__ __forceinline__ T load_chunk(const T* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// acc + q.k over one 16-byte chunk.
template <bool BF16>
__device__ __forceinline__ float dot16(float acc, const u32x4& q, const u32x4& k) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // copy the element out first: a bit-cast of a vector-element lvalue reads element 0
      const unsigned int kw = k[i], qw = q[i];
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw),
                                           __builtin_bit_cast(bf16x2, qw), acc, false);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(q[i]), __uint_as_float(k[i]), acc);
  }
  return acc;
}

// A lane's chunk of a V row -> 8 (bf16, E4M3) or 4 (f32) floats, exactly.
template <int ET, class T>
__device__ __forceinline__ void unpack_chunk(const T& c, float* v) {
  if constexpr (ET == kFP8) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const unsigned int word = c[w];  // codes of 4 consecutive elements, lowest byte first
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
      v[4 * w] = lo[0];
      v[4 * w + 1] = lo[1];
      v[4 * w + 2] = hi[0];
      v[4 * w + 3] = hi[1];
    }
  } else if constexpr (ET == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(c[i] << 16);
      v[2 * i + 1] = __uint_as_float(c[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(c[i]);
  }
}

// A lane's chunk of a K row in the form it is scored in: bf16 pairs for bf16
// and E4M3 caches (every E4M3 value is a bf16 value; gfx950 converts a pair of
// codes to a bf16 pair in one instruction, exactly with scale 1), f32 for f32
// caches.
template <int ET, class T>
__device__ __forceinline__ u32x4 score_chunk(const T& c) {
  if constexpr (ET == kFP8) {
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const unsigned int word = c[w];
      r[2 * w] = __builtin_bit_cast(unsigned int,
                                    __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false));
      r[2 * w + 1] = __builtin_bit_cast(unsigned int,
                                        __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true));
    }
    return r;
  } else {
    return c;
  }
}

// binary32 -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// First block of a sequence of `len` tokens that a window of W tokens (W > 0)
// reaches: its units are blocks first .. ceil(len / bs) - 1.
__device__ __forceinline__ int window_first_block(int len, int window, int bs) {
  return window > 0 && len > window ? (len - window) / bs : 0;
}

// Workgroup that processes unit u when `total` units are split evenly over
// `groups` workgroups (workgroup g takes [g*total/groups, (g+1)*total/groups)).
__device__ __forceinline__ int group_of_unit(int64_t u, int64_t total, int64_t groups) {
  return int(((u + 1) * groups + total - 1) / total - 1);
}

}  // namespace dev

#ifndef PA_PACE
#define PA_PACE 1  // 0: no issue-priority pacing between the waves of a SIMD
#endif

#ifndef PA_DECODE_MFMA_PV
#define PA_DECODE_MFMA_PV 1  // 1: the MFMA path's P.V on MFMA too; 0: on the VALU
#endif

typedef short v4s __attribute__((ext_vector_type(4)));
#define PA_LDS_PTR(T) __attribute__((address_space(3))) T*

#ifndef PA_MFMA_SCORES
#define PA_MFMA_SCORES 1  // 0: score every case on the VALU (for comparison)
#endif

// Scores on the matrix cores: bf16 and 8-bit caches with 128-dim heads and
// blocks of at least 16 rows (an MFMA tile is 16 rows of one block).
constexpr bool decode_uses_mfma(int et, int d, int bs) {
  return PA_MFMA_SCORES && et != kF32 && (d == 128 || (d == 64 && PA_DECODE_MFMA_PV)) &&
         bs >= 8;
}

// LDS bytes each wave of the MFMA path uses: a 16-row K tile padded to 17
// chunks per row (conflict-free transposed reads), the softmax weights
// [4 row groups][G heads][4 rows], the rescale factors [4][G], and the G
// query rows of the sequence being scored (16 chunks of 16 bytes each).
constexpr int decode_wave_lds_bytes(int et, int d, int g, int bs) {
  return decode_uses_mfma(et, d, bs) ? 16 * (d / 8 + 1) * 16 + 64 * g + 16 * g + (d / 8) * 16 * g
                                     : 0;
}

// Byte offset of the per-wave LDS areas behind the unit prefix (balanced mode).
constexpr size_t decode_prefix_lds_bytes(int num_seqs, bool balanced) {
  return balanced ? (size_t(num_seqs + 1) * 4 + 15) / 16 * 16 : 0;
}

template <int ET, int D, int BS, int G, int PF, bool NT>
__global__ void __launch_bounds__(512) decode_kernel(DecodeArgs a) {
  using namespace dev;
  constexpr bool BF16 = ET != kF32;                  // q, and K as scored, in bf16
  constexpr int EB = ET == kF32 ? 4 : ET == kBF16 ? 2 : 1;  // K/V element bytes
  constexpr int QEB = BF16 ? 2 : 4;                  // q element bytes
  constexpr int LB = ET == kFP8 ? 8 : 16;            // bytes a lane loads per row chunk
  using Raw = typename LaneChunk<LB>::type;
  constexpr int VEC = LB / EB;                       // elements per lane chunk
  constexpr int LPR = D / VEC;                       // lanes per row
  constexpr int RPI = 64 / LPR;                      // rows per load instruction
  constexpr bool MF = decode_uses_mfma(ET, D, BS);   // q.k on MFMA (16-row tiles)
  constexpr int QCH = D / 8;                         // 16-byte chunks of a bf16 query row
  constexpr int KCH = D / 8 + 1;                     // 16-byte chunks of an LDS tile row (padded)
  constexpr int MM = D / 32;                         // score MFMAs per tile
  constexpr int QC = MF ? (QCH * G + 63) / 64 : 1;   // query chunks a lane loads per tile
  constexpr int TRW = MF ? 16 : (G > 4 ? 2 : 4) * RPI;   // wide groups keep smaller tiles
  constexpr int TR = MF ? 16 : BS < TRW ? BS : TRW;  // rows per register tile
  constexpr int NI = TR / RPI;                       // load instructions per tile
  // A unit is BPT consecutive blocks of one sequence: one block, or on the
  // MFMA path with 8-token blocks a pair of them filling one 16-row tile
  // (rows 0..7 from the first block, 8..15 from the second).
  constexpr int BPT = TR > BS ? TR / BS : 1;         // blocks per unit
  constexpr int TPB = BPT > 1 ? 1 : BS / TR;         // tiles per unit
  constexpr int NB = PF + 1;                         // ring buffers
  static_assert(D % VEC == 0 && 64 % LPR == 0 && TR % RPI == 0, "tiling");
  static_assert(BPT == 1 ? BS % TR == 0 : (MF && BPT == 2), "a unit is one block or an MFMA pair");
  static_assert(RPI * D * EB == 64 * LB, "one load instruction covers whole rows");
  static_assert(!BF16 || VEC == 8, "bf16 query chunks hold 8 elements");
  static_assert(!MF || (TR == 16 && NI * RPI == 16 && MM % 2 == 0),
                "MFMA tiles are 16 rows: NI consecutive rows per row group");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwave = blockDim.x >> 6;
  const int r = lane / LPR;
  const int c = lane % LPR;
  const int kvh = blockIdx.y * nwave + wave;
  const int head0 = kvh * G;
  const int max_tokens = a.max_blocks * BS;

  // ---- the unit range [ubeg, uend) of this workgroup -----------------------
  // Units are (sequence, block) pairs.  In single and partition modes they
  // all belong to one sequence `fixed_seq` and unit index = block index.
  extern __shared__ int32_t s_prefix[];
  __shared__ int32_t s_prog[8];  // tiles done by each wave (issue pacing)
  if (threadIdx.x < 8) s_prog[threadIdx.x] = 0;
  int fixed_seq = -1;
  int64_t ubeg, uend;
  // single and partition modes: unit uu starts at block fix_blk0 + BPT * uu and
  // the walk's blocks end at fix_bend (units are block indices when BPT = 1)
  int fix_blk0 = 0, fix_bend = 0;
  int64_t total_units = 0, num_groups = 0;
  if (a.mode == kModeBalanced) {
    const int S = a.num_seqs;
    for (int i = threadIdx.x; i < S; i += blockDim.x) {
      int len = a.context_lens[i];
      len = len < 0 ? 0 : (len > max_tokens ? max_tokens : len);
      s_prefix[i + 1] =
          ((len + BS - 1) / BS - window_first_block(len, a.window, BS) + BPT - 1) / BPT;
    }
    if (threadIdx.x == 0) s_prefix[0] = 0;
    __syncthreads();
    if (wave == 0) {
      int carry = 0;
      for (int base = 0; base < S; base += 64) {
        const int i = base + lane;
        const int v = wave_inclusive_sum(i < S ? s_prefix[i + 1] : 0);
        if (i < S) s_prefix[i + 1] = carry + v;
        carry += __builtin_amdgcn_readlane(v, 63);
      }
    }
    __syncthreads();
    total_units = s_prefix[S];
    // never more workgroups than units, so no workgroup's range is empty and
    // the pieces of a sequence come from consecutive workgroups g0..g1
    num_groups = min(int64_t(a.num_groups), total_units);
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      for (int i = threadIdx.x; i <= S; i += blockDim.x) a.info[2 + i] = s_prefix[i];
      if (threadIdx.x == 0) {
        a.info[0] = int32_t(num_groups);
        a.info[1] = int32_t(total_units);
      }
    }
    ubeg = blockIdx.x < num_groups ? int64_t(blockIdx.x) * total_units / num_groups : 0;
    uend = blockIdx.x < num_groups ? int64_t(blockIdx.x + 1) * total_units / num_groups : 0;
  } else {
    __syncthreads();  // s_prog
    fixed_seq = a.mode == kModeSingle ? blockIdx.x : blockIdx.z;
    int len = a.context_lens[fixed_seq];
    len = len < 0 ? 0 : (len > max_tokens ? max_tokens : len);
    const int nblk = (len + BS - 1) / BS;
    ubeg = window_first_block(len, a.window, BS);  // (partition mode has no window)
    uend = nblk;
    if (a.mode == kModePartition) {
      ubeg = int64_t(blockIdx.x) * a.partition_blocks;
      uend = min(int64_t(nblk), ubeg + a.partition_blocks);
      if (ubeg >= uend) return;  // whole workgroup, before any barrier
    }
    fix_bend = int(uend);
    if constexpr (BPT > 1) {
      fix_blk0 = int(ubeg);
      uend = (uend - ubeg + BPT - 1) / BPT;
      ubeg = 0;
    }
  }

  // Per-wave LDS of the MFMA path, behind the unit prefix.
  uint8_t* wave_lds = reinterpret_cast<uint8_t*>(s_prefix) +
                      decode_prefix_lds_bytes(a.num_seqs, a.mode == kModeBalanced) +
                      size_t(wave) * decode_wave_lds_bytes(ET, D, G, BS);
  u32x4* lds_k = reinterpret_cast<u32x4*>(wave_lds);              // [16 rows][KCH chunks]
  float* lds_p = reinterpret_cast<float*>(wave_lds + 16 * KCH * 16);  // [4][G][4]
  float* lds_a = lds_p + 16 * G;                                   // [4][G]
  u32x4* lds_q = reinterpret_cast<u32x4*>(lds_a + 4 * G);          // [G][16 chunks]

  const size_t head_bytes = size_t(BS) * D * EB;
  const size_t block_bytes = head_bytes * a.num_kv_heads;
  const uint8_t* kbase = a.k_pool + kvh * head_bytes;
  const uint8_t* vbase = a.v_pool + kvh * head_bytes;
  const float cl2 = a.k_scales ? a.scale_log2 * a.k_scales[kvh] : a.scale_log2;
  const float vsc = a.v_scales ? a.v_scales[kvh] : a.v_scale;
  // ALiBi slopes in log2 units: the MFMA path's lane 16g + h scores head h
  // (lanes past G repeat a head whose column is never used); the VALU path
  // keeps all G of its group.
  float alibi2 = 0.f;
  float alibi2h[G];
#pragma unroll
  for (int h = 0; h < G; ++h) alibi2h[h] = 0.f;
  if (a.alibi) {
    constexpr float kLog2e = 1.4426950408889634f;
    if constexpr (MF) {
      alibi2 = a.alibi[head0 + min(lane & 15, G - 1)] * kLog2e;
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) alibi2h[h] = a.alibi[head0 + h] * kLog2e;
    }
  }

  // Single pass over an empty sequence: the output is zero.
  if (a.mode == kModeSingle && uend == 0) {
    if (r == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const size_t idx = (size_t(fixed_seq) * a.num_heads + head0 + h) * D + c * VEC;
        if (a.out_f32) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) static_cast<float*>(a.out)[idx + e] = 0.f;
        } else {
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + idx) = u32x4{0, 0, 0, 0};
        }
      }
    }
    return;
  }

  // ---- per-piece state -------------------------------------------------------
  // Row group r = lane / LPR accumulates, for its D/LPR dims, the rows it sees.
  // VALU path: every lane of a group keeps the group's running max m and sum l
  // for all G heads.  MFMA path: lane 16g + h (h < G) keeps them for group g,
  // head h in mf_m / mf_l; m[] and l[] are filled only when a piece is emitted.
  float m[G], l[G], acc[G][VEC];
  float mf_m = kNegInf, mf_l = 0.f;
  // MFMA P.V: O^T blocks of 16 dims (lane 16g + h: dims 16b + 4g + v of
  // head h), the exponent base mf_m (shared by the four row groups of a head
  // and moved lazily) and the true running maximum mf_top
  constexpr bool MFPV = MF && PA_DECODE_MFMA_PV;
  constexpr int NB16 = D / 16;
  f32x4 oacc[MFPV ? NB16 : 1];
  float mf_top = kNegInf;
  u32x4 qc[MF ? 1 : G];  // VALU path: chunk c of each head's query
  u32x4 qf[MF ? MM : 1];  // MFMA path: the current sequence's query as B operands

  // Emit the finished piece of sequence `seq`: the final output when the piece
  // is the whole sequence, else a partial row.
  auto emit = [&](int seq, bool whole) {
    if constexpr (MFPV) {
      // the four row groups' sums share the base; the maximum and the sum are
      // reported against the true maximum
      const float lt = xor_sum<16>(mf_l);
      const int hh = lane & 15;
      if (hh < G) {
        const float inv = lt > 0.f ? vsc / lt : 0.f;
        const int head = head0 + hh;
        const int d0 = 4 * (lane >> 4);
        if (whole) {
          const size_t idx = (size_t(seq) * a.num_heads + head) * D + d0;
          // Every value is computed before the first store.  The temporaries
          // may reuse registers of a tile whose loads the compiler still counts
          // as pending, and a wait for those issued after a store also waits
          // for the next tile's loads, which were issued before that store.
          if (a.out_f32) {
            f32x4 o[NB16];
#pragma unroll
            for (int b = 0; b < NB16; ++b) o[b] = oacc[b] * inv;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < NB16; ++b)
              *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + idx + 16 * b) = o[b];
          } else {
            u32x2 w[NB16];
#pragma unroll
            for (int b = 0; b < NB16; ++b) {
              const f32x4 o = oacc[b] * inv;
              w[b] = u32x2{to_bf16(o[0]) | (to_bf16(o[1]) << 16),
                           to_bf16(o[2]) | (to_bf16(o[3]) << 16)};
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < NB16; ++b)
              *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + idx + 16 * b) = w[b];
          }
        } else {
          size_t row;
          if (a.mode == kModePartition)
            row = (size_t(seq) * a.num_heads + head) * a.max_parts + blockIdx.x;
          else
            row = (size_t(blockIdx.x) + seq) * a.num_heads + head;  // piece slot g + seq
          float* o = a.part_out + row * D + d0;
          // (all values before the first store, as above)
          f32x4 ov[NB16];
#pragma unroll
          for (int b = 0; b < NB16; ++b) ov[b] = oacc[b] * inv;
          const float lsum = mf_top == kNegInf ? 0.f : lt * fast_exp2(mf_m - mf_top);
          // partition partials carry natural-log maxima; pieces stay in log2 units
          const float mx = (mf_top == kNegInf || a.mode == kModeBalanced) ? mf_top
                                                                          : mf_top * kLn2;
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int b = 0; b < NB16; ++b) *reinterpret_cast<f32x4*>(o + 16 * b) = ov[b];
          if (lane < 16) {
            a.part_max[row] = mx;
            a.part_sum[row] = lsum;
          }
        }
      }
      return;
    }
    if constexpr (MF) {
      // hand each row group's (m, l) of every head to all lanes of the group
      if ((lane & 15) < G) {
        lds_p[(lane >> 4) * G + (lane & 15)] = mf_m;
        lds_p[4 * G + (lane >> 4) * G + (lane & 15)] = mf_l;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m[h] = lds_p[r * G + h];
        l[h] = lds_p[4 * G + r * G + h];
      }
      __builtin_amdgcn_wave_barrier();
    }
    // merge the RPI row groups (lanes that differ in r)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float big = xor_max<LPR>(m[h]);
      const float f = (m[h] == kNegInf) ? 0.f : fast_exp2(m[h] - big);
      const float lw = xor_sum<LPR>(l[h] * f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = xor_sum<LPR>(acc[h][e] * f);
      m[h] = big;
      l[h] = lw;
    }
    if (r != 0) return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = l[h] > 0.f ? vsc / l[h] : 0.f;
      const int head = head0 + h;
      if (whole) {
        const size_t idx = (size_t(seq) * a.num_heads + head) * D + c * VEC;
        if (a.out_f32) {
          float* o = static_cast<float*>(a.out) + idx;
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[e] = acc[h][e] * inv;
        } else {
          u32x4 packed;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            packed[i] = to_bf16(acc[h][2 * i] * inv) | (to_bf16(acc[h][2 * i + 1] * inv) << 16);
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + idx) = packed;
        }
      } else {
        size_t row;
        if (a.mode == kModePartition)
          row = (size_t(seq) * a.num_heads + head) * a.max_parts + blockIdx.x;
        else
          row = (size_t(blockIdx.x) + seq) * a.num_heads + head;  // piece slot g + seq
        float* o = a.part_out + row * D + c * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = acc[h][e] * inv;
        if (c == 0) {
          // partition partials carry natural-log maxima; pieces stay in log2 units
          const float mx = (m[h] == kNegInf || a.mode == kModeBalanced) ? m[h] : m[h] * kLn2;
          a.part_max[row] = mx;
          a.part_sum[row] = l[h];
        }
      }
    }
  };

  // ---- the walk: one ring of tiles over the whole unit range -----------------
  // Units are taken in order; a piece is a maximal run of them that shares a
  // sequence.  The ring of register tiles runs across piece boundaries: the
  // next piece's first tiles, its query and the next 64 block-table entries
  // are in flight before the current piece ends.  The steady-state loop issues
  // the same loads every iteration (no tile load sits behind a branch), so the
  // compiler's wait before scoring a tile leaves the later tiles' loads in
  // flight; prefetches past the range, and tiles whose table entry is out of
  // range, read block 0 instead (their data is never used).
  if (ubeg >= uend) return;  // balanced mode: workgroups past the unit count
  const int ntiles = int(uend - ubeg) * TPB;

  // Sequence holding unit uu (balanced mode): s_prefix[seq] <= uu < s_prefix[seq + 1].
  auto seq_of = [&](int64_t uu) {
    int lo = 0, hi = a.num_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_prefix[mid] <= uu) lo = mid; else hi = mid;
    }
    return lo;
  };

  // A window describes 64 consecutive units; lane k holds, for unit
  // cbase + k, its sequence (sk), its block index in the sequence (jk), the
  // raw table entry (ek) and the sequence's raw context length (lk).  Lanes
  // past the range repeat the range's last unit, so every lane loads and the
  // loads write the window's registers directly; entries and lengths are
  // checked where they are used.
  // With block pairs (BPT = 2), jk is the pair's first block and ek2 the
  // second block's entry, or -1 when the walk ends at the first.
  struct Window {
    int ek, lk, jk, sk, ek2;
  };
  auto fetch_window = [&](int64_t cbase) {
    const int64_t uu = min(cbase + lane, uend - 1);
    Window w;
    if (fixed_seq >= 0) {
      w.sk = fixed_seq;
      w.lk = a.context_lens[w.sk];
      w.jk = fix_blk0 + BPT * int(uu);
    } else {
      w.sk = seq_of(uu);
      w.lk = a.context_lens[w.sk];
      w.jk = BPT * int(uu - s_prefix[w.sk]);
      if (a.window > 0) {  // only then does the table entry's index wait for the length
        const int len = w.lk < 0 ? 0 : (w.lk > max_tokens ? max_tokens : w.lk);
        w.jk += window_first_block(len, a.window, BS);
      }
    }
    const int32_t* trow = a.block_tables + size_t(w.sk) * a.max_blocks;
    w.ek = trow[w.jk];
    w.ek2 = -1;
    if constexpr (BPT > 1) {
      // the second block's entry is read only when the walk reaches it
      int bend = fix_bend;
      if (fixed_seq < 0) {
        const int len = w.lk < 0 ? 0 : (w.lk > max_tokens ? max_tokens : w.lk);
        bend = (len + BS - 1) / BS;
      }
      if (w.jk + 1 < bend) w.ek2 = trow[w.jk + 1];
    }
    return w;
  };

  // Query registers of sequence sq (MFMA path: lane 16g + h holds head h's
  // dims [32mm + 8g, 32mm + 8g + 8) of MFMA mm, lanes with h >= G a copy of a
  // real head whose score column is never used; VALU path: chunk c of each
  // head).  Every lane loads, so the registers are written by the loads alone.
  auto load_q = [&](int sq, u32x4(&dqc)[MF ? 1 : G], u32x4(&dqf)[MF ? 4 : 1]) {
    const u32x4* qrow =
        reinterpret_cast<const u32x4*>(a.q + (size_t(sq) * a.num_heads + head0) * D * QEB);
    if constexpr (MF) {
      const int h = (lane & 15) % G;
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) dqf[mm] = qrow[h * QCH + 4 * mm + (lane >> 4)];
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) dqc[h] = qrow[h * LPR + c];
    }
  };

  auto reset_state = [&]() {
    mf_m = kNegInf;
    mf_l = 0.f;
    mf_top = kNegInf;
    if constexpr (MFPV) {
#pragma unroll
      for (int b = 0; b < NB16; ++b) oacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
    }
  };

  // current piece: units [pstart, pend) of sequence seq; `whole` when it is
  // all of the sequence (balanced mode).  sq is unit uu's sequence, taken from
  // the table-entry window that covers uu (no search of the prefix).
  int seq;
  int64_t pstart, pend;
  bool whole;
  // a piece that ended and is closed at the start of the next step
  bool closing = false;
  int64_t close_at = 0;
  int close_sq = 0;
  auto start_piece = [&](int64_t uu, int sq) {
    if (fixed_seq >= 0) {
      seq = fixed_seq;
      pend = uend;
      whole = a.mode == kModeSingle;
    } else {
      seq = sq;
      const int64_t first = s_prefix[seq], last = s_prefix[seq + 1];
      pend = min(uend, last);
      whole = uu == first && pend == last;
    }
    pstart = uu;
  };

  // Windows of units [cbase, +64) and [+64, +128); tiles at most PF ahead of
  // the current one fall in one of them.
  int64_t cbase = ubeg;
  Window w0 = fetch_window(cbase);
  Window w1 = fetch_window(cbase + 64);

  // Fused append, part 1: each wave writes the new token's K and V rows of its
  // KV head for every sequence whose last block is one of this workgroup's
  // units.  The input rows of the first two such sequences are loaded here,
  // ahead of the first tiles, so writing them later waits for no tile.  Lanes
  // 0..31 handle K, 32..63 V, one 16-byte input chunk each.
  const bool appending = a.k_new != nullptr && a.mode != kModePartition;
  constexpr int kAppChunks = D * QEB / 16;  // 16-byte chunks of an input row
  const bool app_v = lane >= 32;
  const int app_ch = lane & 31;
  // The K-or-V choice of a lane is an offset from the K pointer (a per-lane
  // choice between two argument fields would be a per-lane memory load); lanes
  // past the row read its last chunk again, so every lane loads.
  const int64_t app_src_off = app_v ? a.v_new - a.k_new : 0;
  const int64_t app_pool_off = app_v ? a.v_pool - a.k_pool : 0;
  const float app_kenc = appending && a.k_scales ? a.k_scales[kvh] : a.k_enc;
  const float app_venc = appending && a.v_scales ? a.v_scales[kvh] : a.v_enc;
  const uint32_t app_scale = app_v ? __builtin_amdgcn_readfirstlane(__float_as_uint(app_venc))
                                   : __builtin_amdgcn_readfirstlane(__float_as_uint(app_kenc));
  const int app_chl = app_ch < kAppChunks ? app_ch : kAppChunks - 1;
  auto new_chunk = [&](int sq) {
    return reinterpret_cast<const uint4*>(a.k_new + app_src_off +
                                          (size_t(sq) * a.num_kv_heads + kvh) * D * QEB)[app_chl];
  };
  int app_seq[2] = {-1, -1};
  int64_t app_last[2] = {0, 0};
  uint4 app_in[2];
  int app_resume = a.num_seqs;
  if (appending) {
    if (fixed_seq >= 0) {
      app_seq[0] = fixed_seq;
      app_last[0] = uend - 1;
    } else {
      int k = 0, sq = seq_of(ubeg);
      for (; sq < a.num_seqs && k < 2; ++sq) {
        const int64_t last = int64_t(s_prefix[sq + 1]) - 1;
        if (last >= uend) break;
        if (s_prefix[sq + 1] > s_prefix[sq] && last >= ubeg) {
          app_seq[k] = sq;
          app_last[k] = last;
          ++k;
        }
      }
      app_resume = sq;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (app_seq[k] >= 0) app_in[k] = new_chunk(app_seq[k]);
  }
  start_piece(ubeg, __builtin_amdgcn_readlane(w0.sk, 0));
  // VALU path: the current piece's query and the next piece's, swapped at a
  // piece boundary.  (The MFMA path carries the query in the tile ring.)
  u32x4 qc_next[MF ? 1 : G];
  if constexpr (!MF) {
    load_q(seq, qc, qf);
    load_q(pend < uend ? __builtin_amdgcn_readfirstlane(seq_of(pend)) : seq, qc_next, qf);
  }
  reset_state();

  // Loads tile t into (kr, vr).  On the MFMA path a tile that starts a new
  // sequence in the walk also brings the G query rows of that sequence in qr
  // (one 16-byte chunk per lane, QC per lane for G = 8): the query arrives in
  // the ring with the first tile it is scored against, so a piece boundary
  // needs no separate query load, and other tiles load no query at all.
  int q_loaded = -1;     // sequence of the last query loaded into the ring
  int q_staged = -1;     // sequence whose query rows sit in lds_q
  auto load_tile = [&](Raw(&kr)[NI], Raw(&vr)[NI], u32x4(&qr)[QC], int t) {
    int phys = -1, phys2 = -1, sq = 0;
    size_t off = 0;
    if (t < ntiles) {
      const int idx = int(ubeg + t / TPB - cbase);  // < 128: at most PF tiles ahead
      if (idx < 64) {
        phys = __builtin_amdgcn_readlane(w0.ek, idx);
        sq = __builtin_amdgcn_readlane(w0.sk, idx);
        if constexpr (BPT > 1) phys2 = __builtin_amdgcn_readlane(w0.ek2, idx);
      } else {
        phys = __builtin_amdgcn_readlane(w1.ek, idx - 64);
        sq = __builtin_amdgcn_readlane(w1.sk, idx - 64);
        if constexpr (BPT > 1) phys2 = __builtin_amdgcn_readlane(w1.ek2, idx - 64);
      }
      off = size_t(t % TPB) * (TR * D * EB);
    }
    if constexpr (MF) {
      if (t < ntiles && sq != q_loaded) {
        q_loaded = sq;
        const u32x4* qrow =
            reinterpret_cast<const u32x4*>(a.q + (size_t(sq) * a.num_heads + head0) * D * QEB);
#pragma unroll
        for (int j = 0; j < QC; ++j) {
          const int ch = lane + 64 * j;
          qr[j] = qrow[ch < QCH * G ? ch : ch % (QCH * G)];  // lanes past the rows repeat one
        }
      }
    }
    if (phys < 0 || int64_t(phys) >= a.num_blocks) {
      phys = 0;
      off = 0;
    }
    off += size_t(phys) * block_bytes;
    // VALU path: instruction i holds rows i*RPI + r.  MFMA path: rows 4r + i,
    // so each row group sees 4 consecutive rows, as the MFMA result rows.
    // (Every instruction reads 1 KiB of whole rows; loading K straight in
    // the MFMA operand layout instead - 64-byte pieces of 16 rows - was
    // measured slower than transposing it through LDS.)  With block pairs,
    // row groups 2 and 3 read rows 0..7 of the second block.
    int lo = MF ? NI * LPR * r + c : lane;
    if constexpr (BPT > 1) {
      if (phys2 < 0 || int64_t(phys2) >= a.num_blocks) phys2 = 0;
      if (NI * r >= 8) {
        off = size_t(phys2) * block_bytes;
        lo -= 8 * LPR;
      }
    }
    constexpr int step = MF ? LPR : 64;
    const Raw* kp = reinterpret_cast<const Raw*>(kbase + off) + lo;
    const Raw* vp = reinterpret_cast<const Raw*>(vbase + off) + lo;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      kr[i] = load_chunk<NT>(kp + i * step);
      vr[i] = load_chunk<NT>(vp + i * step);
    }
  };

  auto process_tile = [&](const Raw(&kr)[NI], const Raw(&vr)[NI], const u32x4(&qr)[QC],
                          int t) {
    const int idx = int(ubeg + t / TPB - cbase);
    const int phys = __builtin_amdgcn_readlane(w0.ek, idx);
    int len = __builtin_amdgcn_readlane(w0.lk, idx);
    len = len < 0 ? 0 : (len > max_tokens ? max_tokens : len);
    const int tok0 = __builtin_amdgcn_readlane(w0.jk, idx) * BS + (t % TPB) * TR;
    const bool ok1 = phys >= 0 && int64_t(phys) < a.num_blocks;
    int nvalid = min(TR, len - tok0);
    // rows before a sliding window (positions < len - W) are masked like the
    // rows past the end
    int nskip = a.window > 0 ? max(0, len - a.window - tok0) : 0;
    if constexpr (BPT > 1) {
      // a pair: a first block outside the pool masks rows 0..7, a missing or
      // bad second block rows 8..15
      const int phys2 = __builtin_amdgcn_readlane(w0.ek2, idx);
      if (!(phys2 >= 0 && int64_t(phys2) < a.num_blocks)) nvalid = min(nvalid, BS);
      if (!ok1) nskip = max(nskip, BS);
    } else {
      if (!ok1) nvalid = 0;
    }
    if constexpr (MF) {
      // The first tile of a sequence brought its query rows (see load_tile):
      // they go through LDS into the B layout once, and stay in qf after -
      // also when that tile itself contributes nothing.
      const int tseq = __builtin_amdgcn_readlane(w0.sk, idx);
      if (tseq != q_staged) {
        q_staged = tseq;
#pragma unroll
        for (int j = 0; j < QC; ++j)
          if (lane + 64 * j < QCH * G) lds_q[lane + 64 * j] = qr[j];
        __builtin_amdgcn_wave_barrier();
        const int qh = (lane & 15) % G;
#pragma unroll
        for (int mm = 0; mm < MM; ++mm) qf[mm] = lds_q[qh * QCH + 4 * mm + (lane >> 4)];
      }
    }
    // Every row masked: the state would not change.  The VALU path skips the
    // tile; the MFMA path runs it like any other (all its weights are zero,
    // its V rows are zeroed, and the state comes out bit for bit the same),
    // so that every path through here has read the tile's registers: code
    // after this tile may reuse them, and a wait for their loads there would
    // come after the next tile's loads were issued and stall until they return.
    if (!MF && nvalid <= nskip) return;
    const bool partial = nvalid < TR || nskip > 0;
    if constexpr (MF) {
      // K tile -> LDS, then read back transposed: lane 16g + t gets row t's
      // dims [32mm + 8g, 32mm + 8g + 8) as the A operand of MFMA mm, and lane
      // 16g + h holds the same dims of query head h as B (h < G; the other
      // lanes repeat a head whose score column is never used).
#pragma unroll
      for (int i = 0; i < NI; ++i) lds_k[(NI * r + i) * KCH + c] = score_chunk<ET>(kr[i]);
      // two independent accumulation chains of two MFMAs each
      f32x4 sc_even = {0.f, 0.f, 0.f, 0.f}, sc_odd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mm = 0; mm < MM; mm += 2) {
        const u32x4 ka = lds_k[(lane & 15) * KCH + 4 * mm + (lane >> 4)];
        const u32x4 kb2 = lds_k[(lane & 15) * KCH + 4 * (mm + 1) + (lane >> 4)];
        sc_even = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, ka), __builtin_bit_cast(bf16x8, qf[mm]), sc_even, 0, 0, 0);
        sc_odd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, kb2), __builtin_bit_cast(bf16x8, qf[mm + 1]), sc_odd, 0,
            0, 0);
      }
      const f32x4 sc = sc_even + sc_odd;
      // lane 16g + h: scores of rows 4g + v (v = 0..3), head h
      const int g4 = 4 * (lane >> 4);
      float sv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) sv[v] = sc[v] * cl2;
      if (a.alibi) {  // slope * (position - (len - 1)), in log2 units
        const float d0 = float(tok0 + g4 - (len - 1));
#pragma unroll
        for (int v = 0; v < 4; ++v) sv[v] = fmaf(alibi2, d0 + float(v), sv[v]);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (partial && (g4 + v >= nvalid || g4 + v < nskip)) sv[v] = kNegInf;
      if constexpr (MFPV) {
        // One base per head over its four row groups (lanes h, 16+h, 32+h,
        // 48+h).  It moves only when the maximum passes it by more than 8
        // (log2 units): weights stay <= 2^8 and O is rescaled rarely.
        const float mx = xor_max<16>(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
        mf_top = fmaxf(mf_top, mx);
        const bool move = mx > mf_m + 8.f;
        const float mnew = move ? mx : mf_m;
        const float base = (mnew == kNegInf) ? 0.f : mnew;
        const float alpha = move ? fast_exp2(mf_m - base) : 1.f;
        mf_m = mnew;
        float pv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) pv[v] = fast_exp2(sv[v] - base);
        mf_l = fmaf(mf_l, alpha, (pv[0] + pv[1]) + (pv[2] + pv[3]));
        if (__ballot(move) != 0) {
#pragma unroll
          for (int b = 0; b < NB16; ++b) oacc[b] *= alpha;
        }
        // The weights of rows 4g..4g+3 of head h, already in lane 16g + h, are
        // the B operand of O^T += V^T P, as three bf16 terms: the weight's top
        // 16 bits, then those of each remainder (both subtractions are exact);
        // together they leave out less than 2^-23 of the weight.
        v4s p3[3];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float rest = pv[v];
#pragma unroll
          for (int k = 0; k < 3; ++k) {
            const uint32_t top = __float_as_uint(rest) & 0xFFFF0000u;
            p3[k][v] = short(top >> 16);
            rest -= __uint_as_float(top);
          }
        }
        // V tile -> LDS over the K tile just read (row-major, 17 chunks a row),
        // rows that do not count zeroed (they may hold NaN); then transposed
        // reads give lane 16g + s dim 16b + s of rows 4g..4g+3: the A operand.
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          u32x4 vc = score_chunk<ET>(vr[i]);
          if (partial && (NI * r + i >= nvalid || NI * r + i < nskip)) vc = u32x4{0u, 0u, 0u, 0u};
          lds_k[(NI * r + i) * KCH + c] = vc;
        }
        asm volatile("" ::: "memory");
        PA_LDS_PTR(uint8_t) lv = (PA_LDS_PTR(uint8_t))lds_k;
        const int voff = (4 * (lane >> 4) + ((lane & 15) >> 2)) * (KCH * 16) + 8 * (lane & 3);
#pragma unroll
        for (int b = 0; b < NB16; ++b) {
          const v4s vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS_PTR(v4s))(lv + voff + 32 * b));
#pragma unroll
          for (int k = 0; k < 3; ++k)
            oacc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, p3[k], oacc[b], 0, 0, 0);
        }
        asm volatile("" ::: "memory");
        return;
      }
      const float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      const float mnew = fmaxf(mf_m, mx);
      const float base = (mnew == kNegInf) ? 0.f : mnew;
      const float alpha = fast_exp2(mf_m - base);
      float pv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) pv[v] = fast_exp2(sv[v] - base);
      mf_l = fmaf(mf_l, alpha, (pv[0] + pv[1]) + (pv[2] + pv[3]));
      mf_m = mnew;
      const bool live = (lane & 15) < G;
      if (live) {
        float* dst = lds_p + ((lane >> 4) * G + (lane & 15)) * 4;
#pragma unroll
        for (int v = 0; v < 4; ++v) dst[v] = pv[v];
        lds_a[(lane >> 4) * G + (lane & 15)] = alpha;
      }
      const bool rescale = __ballot(live && alpha != 1.f) != 0;
      __builtin_amdgcn_wave_barrier();
      // row group r reads its weights: rows 4r + i, every head
      if (rescale) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float al = lds_a[r * G + h];
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[h][e] *= al;
        }
      }
      float v[4][VEC];
#pragma unroll
      for (int i = 0; i < 4; ++i) unpack_chunk<ET>(vr[i], v[i]);
      if (__builtin_expect(partial, 0)) {  // the last block of a sequence only
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * r + i >= nvalid || 4 * r + i < nskip)
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[i][e] = 0.f;  // masked rows may hold NaN
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ph = lds_p[(r * G + h) * 4 + i];
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(ph, v[i][e], acc[h][e]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    } else {
      float s[NI][G];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h)
          s[i][h] = group_sum<LPR>(dot16<BF16>(0.f, qc[h], score_chunk<ET>(kr[i]))) * cl2;
      if (a.alibi) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const float d = float(tok0 + i * RPI + r - (len - 1));
#pragma unroll
          for (int h = 0; h < G; ++h) s[i][h] = fmaf(alibi2h[h], d, s[i][h]);
        }
      }
      if (partial) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
          if (i * RPI + r >= nvalid || i * RPI + r < nskip)
#pragma unroll
            for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
      }
      float p[NI][G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = s[0][h];
#pragma unroll
        for (int i = 1; i < NI; ++i) mx = fmaxf(mx, s[i][h]);
        const float mnew = fmaxf(m[h], mx);
        const float base = (mnew == kNegInf) ? 0.f : mnew;
        const float alpha = fast_exp2(m[h] - base);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          p[i][h] = fast_exp2(s[i][h] - base);
          ps += p[i][h];
        }
        l[h] = fmaf(l[h], alpha, ps);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] *= alpha;
        m[h] = mnew;
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float v[VEC];
        unpack_chunk<ET>(vr[i], v);
        if (partial && (i * RPI + r >= nvalid || i * RPI + r < nskip)) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = 0.f;  // masked rows may hold NaN
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(p[i][h], v[e], acc[h][e]);
      }
    }
  };

  // MFMA path: the deferred end of a piece - write it and start the next one.
  auto close_piece = [&]() {
    closing = false;
    emit(seq, whole);
    start_piece(close_at, close_sq);
    reset_state();
  };

  // After the last tile of a unit: close the piece if the unit ended it, and
  // move the table-entry window when the next unit starts a new chunk.
  auto unit_done = [&](int64_t next) {
    if (next == pend) {
      // MFMA path: closing the piece (its output or partial write) waits on
      // the MFMA results and the stores; unless it is the last one, it is done
      // after the next tile's loads are issued (close_piece, at the top of the
      // next step), so that those loads are not held back behind it.
      if (!MF || next == uend) emit(seq, whole);
      if (next < uend) {
        const int idx = int(next - cbase);  // <= 64: the window moves after this
        const int sq = idx < 64 ? __builtin_amdgcn_readlane(w0.sk, idx)
                                : __builtin_amdgcn_readlane(w1.sk, idx - 64);
        if constexpr (MF) {
          close_at = next;
          close_sq = sq;
          closing = true;
        } else {
          start_piece(next, sq);
#pragma unroll
          for (int h = 0; h < G; ++h) qc[h] = qc_next[h];
          load_q(pend < uend ? __builtin_amdgcn_readfirstlane(seq_of(pend)) : seq, qc_next, qf);
          reset_state();
        }
      }
    }
    if (next == cbase + 64) {
      cbase = next;
      w0 = w1;
      w1 = fetch_window(cbase + 64);
    }
  };

  // Issue priority.  An 8-wave workgroup puts waves w and w^4 on one SIMD,
  // where the older wave wins arbitration and would finish its (equal) share
  // well before the younger one, leaving the workgroup waiting on the latter.
  // After each tile a wave publishes its progress and runs at raised priority
  // while it is not ahead of its partner.
  auto pace = [&](int t) {
    if (!PA_PACE || nwave != 8) return;
    s_prog[wave] = t;
    if (t > s_prog[wave ^ 4])
      __builtin_amdgcn_s_setprio(0);
    else
      __builtin_amdgcn_s_setprio(2);
  };

  Raw kb[NB][NI], vb[NB][NI];
  u32x4 qb[NB][QC];
#pragma unroll
  for (int i = 0; i < PF; ++i) load_tile(kb[i], vb[i], qb[i], i);

  // Fused append, part 2 (part 1 loaded the first two rows ahead of the
  // tiles): write the rows, then load and write those of any further
  // sequences.  A wavefront's memory operations take effect in program order
  // and the same wave reads the rows later from its tiles; a row that falls in
  // a tile already in flight has that tile loaded again after the write.
  if (appending) {
    bool reload = false;
    auto write_row = [&](int sq, int64_t last, uint4 in) {
      const int idx = int(last - cbase);
      int phys, len;
      if (idx < 128) {
        const Window& w = idx < 64 ? w0 : w1;
        const int k = idx & 63;
        phys = __builtin_amdgcn_readlane(w.ek, k);
        len = __builtin_amdgcn_readlane(w.lk, k);
        if constexpr (BPT > 1) {
          // the token sits in the pair's second block unless the pair ends early
          const int cl = len < 0 ? 0 : (len > max_tokens ? max_tokens : len);
          if (cl > 0 && (cl - 1) / BS != __builtin_amdgcn_readlane(w.jk, k))
            phys = __builtin_amdgcn_readlane(w.ek2, k);
        }
      } else {  // (scalar results, so no other path waits for these loads)
        len = __builtin_amdgcn_readfirstlane(a.context_lens[sq]);
        const int cl = len < 0 ? 0 : (len > max_tokens ? max_tokens : len);
        phys = cl > 0 ? __builtin_amdgcn_readfirstlane(
                            a.block_tables[size_t(sq) * a.max_blocks + (cl - 1) / BS])
                      : -1;
      }
      len = len < 0 ? 0 : (len > max_tokens ? max_tokens : len);
      if (len == 0 || phys < 0 || int64_t(phys) >= a.num_blocks) return;
      const int pos = len - 1;
      if (int64_t(idx) * TPB + (pos % BS) / TR < PF) reload = true;  // tile already loaded
      if (app_ch >= kAppChunks) return;
      uint8_t* row = const_cast<uint8_t*>(a.k_pool) + app_pool_off + size_t(phys) * block_bytes +
                     kvh * head_bytes + size_t(pos % BS) * D * EB;
      if constexpr (ET == kFP8)
        reinterpret_cast<uint2*>(row)[app_ch] =
            codec::quantize_chunk(in, __uint_as_float(app_scale));
      else
        reinterpret_cast<uint4*>(row)[app_ch] = in;
    };
    if (app_seq[0] >= 0) write_row(app_seq[0], app_last[0], app_in[0]);
    if (app_seq[1] >= 0) write_row(app_seq[1], app_last[1], app_in[1]);
    if (fixed_seq < 0) {
      for (int sq = app_resume; sq < a.num_seqs; ++sq) {
        const int64_t last = int64_t(s_prefix[sq + 1]) - 1;
        if (last >= uend) break;
        if (s_prefix[sq + 1] > s_prefix[sq] && last >= ubeg) write_row(sq, last, new_chunk(sq));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (__builtin_amdgcn_readfirstlane(int(reload))) {
#pragma unroll
      for (int i = 0; i < PF; ++i) load_tile(kb[i], vb[i], qb[i], i);
    }
  }

  for (int t0 = 0; t0 < ntiles; t0 += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int t = t0 + k;
      load_tile(kb[(k + PF) % NB], vb[(k + PF) % NB], qb[(k + PF) % NB], t + PF);
      if (t < ntiles) {
        if constexpr (MF) {
          if (closing) close_piece();
        }
        process_tile(kb[k], vb[k], qb[k], t);
        pace(t);
        if (t % TPB == TPB - 1) unit_done(ubeg + t / TPB + 1);
      }
    }
  }
}

struct MergeArgs {
  const float* piece_out;
  const float* piece_max;
  const float* piece_sum;
  const int32_t* info;
  void* out;
  int32_t num_heads;
  int32_t out_f32;
};

// Merge the pieces of sequences split between workgroups (balanced mode) and
// write zeros for empty sequences.  One wave per (sequence, query head), four
// heads per workgroup.
// After one read of the split description, the pieces' maxima and sums (lane p
// holds piece p) and their output rows (16-byte loads; LR lanes cover a row,
// so one load instruction brings 64/LR pieces) are all in flight at once.
// Pieces are taken 64 at a time with the running log-sum-exp rescale, and
// their rows in batches of NBATCH load instructions.
template <int D>
__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
  using namespace dev;
  constexpr int LR = D / 4;          // lanes per row
  constexpr int PPI = 64 / LR;       // pieces per load instruction
  constexpr int NBATCH = 8;          // load instructions per batch
  constexpr int PB = PPI * NBATCH;   // pieces per batch
  static_assert(64 % LR == 0 && 64 % PB == 0, "merge tiling");
  const int lane = threadIdx.x & 63;
  const int head = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int seq = blockIdx.y;
  if (head >= a.num_heads) return;
  const int sub = lane / LR;         // which piece of an instruction this lane reads
  const int col = (lane % LR) * 4;   // its 4 dims
  const int64_t groups = a.info[0];
  const int64_t total = a.info[1];
  const int64_t u0 = a.info[2 + seq];
  const int64_t u1 = a.info[3 + seq];  // one past the sequence's last unit
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (u1 > u0) {
    const int g0 = group_of_unit(u0, total, groups);
    const int g1 = group_of_unit(u1 - 1, total, groups);
    if (g0 == g1) return;  // one workgroup held the whole sequence and wrote it
    const int np = g1 - g0 + 1;
    const size_t stride = size_t(a.num_heads) * D;  // next workgroup's row of this head
    const float* rows = a.piece_out + ((size_t(g0) + seq) * a.num_heads + head) * D + col;
    const size_t mrow0 = (size_t(g0) + seq) * a.num_heads + head;
    float big = kNegInf;
    for (int p0 = 0; p0 < np; p0 += 64) {
      const int cnt = min(64, np - p0);
      float pm = kNegInf, ps = 0.f;
      if (lane < cnt) {
        const size_t row = mrow0 + size_t(p0 + lane) * a.num_heads;
        ps = a.piece_sum[row];
        pm = a.piece_max[row];
      }
      f32x4 v[NBATCH];
#pragma unroll
      for (int i = 0; i < NBATCH; ++i) {
        const int p = i * PPI + sub;
        v[i] = p < cnt ? *reinterpret_cast<const f32x4*>(rows + size_t(p0 + p) * stride)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const float cmax = wave_max(ps > 0.f ? pm : kNegInf);
      const float nb = fmaxf(big, cmax);
      if (nb != big) {
        const float f = big == kNegInf ? 0.f : fast_exp2(big - nb);
        acc *= f;
        wsum *= f;
        big = nb;
      }
      const float w = ps > 0.f ? ps * fast_exp2(pm - big) : 0.f;
      wsum += wave_sum(w);
      for (int b0 = 0; b0 < cnt; b0 += PB) {
        if (b0 > 0) {
#pragma unroll
          for (int i = 0; i < NBATCH; ++i) {
            const int p = b0 + i * PPI + sub;
            v[i] = p < cnt ? *reinterpret_cast<const f32x4*>(rows + size_t(p0 + p) * stride)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
#pragma unroll
        for (int i = 0; i < NBATCH; ++i) {
          // the weight of piece b0 + i PPI + sub (< 64; lanes past cnt hold
          // w = 0): lane reads of the PPI candidates, no LDS round trip
          float wp = 0.f;
#pragma unroll
          for (int k = 0; k < PPI; ++k) {
            const float c = __uint_as_float(__builtin_amdgcn_readlane(
                __float_as_uint(w), b0 + i * PPI + k));
            wp = sub == k ? c : wp;
          }
          acc += wp * v[i];
        }
      }
    }
    // add up the PPI pieces of each load instruction's lane groups (lane
    // swaps for 16 and 32 lanes apart)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = xor_sum<LR>(acc[e]);
  }
  if (lane >= LR) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const size_t o = (size_t(seq) * a.num_heads + head) * D + col;
  if (a.out_f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o) = acc * inv;
  } else {
    uint16_t* dst = static_cast<uint16_t*>(a.out) + o;
    const uint32_t lo = to_bf16(acc[0] * inv) | (to_bf16(acc[1] * inv) << 16);
    const uint32_t hi = to_bf16(acc[2] * inv) | (to_bf16(acc[3] * inv) << 16);
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  }
}

// Tuning knobs (compile-time): ring depth per group width, widest workgroup.
#ifndef PA_PREFETCH_NARROW
#define PA_PREFETCH_NARROW 1  // tiles in flight ahead of the current one, G <= 4
#endif
#ifndef PA_PREFETCH_WIDE
#define PA_PREFETCH_WIDE 1    // G = 8
#endif
#ifndef PA_PREFETCH_FP8
#define PA_PREFETCH_FP8 1     // 8-bit caches (tiles of half the bytes)
#endif
#ifndef PA_PREFETCH_D64
#define PA_PREFETCH_D64 2     // 64-dim heads, bf16 and f32 caches (tiles of half the bytes)
#endif
#ifndef PA_PREFETCH_D64_FP8
#define PA_PREFETCH_D64_FP8 1 // 64-dim heads, 8-bit caches
#endif
#ifndef PA_MAX_WAVES
#define PA_MAX_WAVES 8        // KV heads (waves) per workgroup at most
#endif

// Tiles in flight ahead of the current one.
constexpr int decode_prefetch(int et, int d, int g) {
  return d == 64 ? (et == kFP8 ? PA_PREFETCH_D64_FP8 : PA_PREFETCH_D64)
         : et == kFP8 ? PA_PREFETCH_FP8
         : g <= 4     ? PA_PREFETCH_NARROW
                      : PA_PREFETCH_WIDE;
}

// Launches decode_kernel for a runtime (D, BS, G) on a grid of `waves`-wave
// workgroups with `lds` bytes of dynamic LDS; false when no instantiation matches.
bool launch_decode_f32(int d, int bs, int g, const DecodeArgs& a, dim3 grid, int waves,
                       size_t lds, hipStream_t s);
bool launch_decode_bf16(int d, int bs, int g, const DecodeArgs& a, dim3 grid, int waves,
                        size_t lds, hipStream_t s);
bool launch_decode_fp8(int d, int bs, int g, const DecodeArgs& a, dim3 grid, int waves,
                       size_t lds, hipStream_t s);

// Workgroups of `waves` waves one CU holds at once for the decode kernel of
// (D, BS, G), or 0 when no instantiation matches.
int decode_groups_per_cu_f32(int d, int bs, int g, int waves, size_t lds);
int decode_groups_per_cu_bf16(int d, int bs, int g, int waves, size_t lds);
int decode_groups_per_cu_fp8(int d, int bs, int g, int waves, size_t lds);

// Query heads per KV head the kernels take: 1..8, and 16 on the MFMA path
// (whose score tile has 16 head columns).
constexpr bool decode_group_supported(int et, int d, int bs, int g) {
  return (g >= 1 && g <= 8) || (g == 16 && decode_uses_mfma(et, d, bs));
}

// Instantiation table: D in {64, 128}, block size in {8, 16, 32}, G in 1..8,
// and G = 16 where the MFMA path runs.
#define PA_DECODE_GROUPS(CASE, D_, BS_)                                                  \
  CASE(D_, BS_, 1) CASE(D_, BS_, 2) CASE(D_, BS_, 3) CASE(D_, BS_, 4) CASE(D_, BS_, 5)  \
  CASE(D_, BS_, 6) CASE(D_, BS_, 7) CASE(D_, BS_, 8)                                    \
  if constexpr (decode_uses_mfma(ET, D_, BS_)) { CASE(D_, BS_, 16) }
#define PA_DECODE_SHAPES(CASE)                                                           \
  PA_DECODE_GROUPS(CASE, 64, 8) PA_DECODE_GROUPS(CASE, 64, 16)                          \
  PA_DECODE_GROUPS(CASE, 64, 32) PA_DECODE_GROUPS(CASE, 128, 8)                         \
  PA_DECODE_GROUPS(CASE, 128, 16) PA_DECODE_GROUPS(CASE, 128, 32)

template <int ET>
bool launch_decode_impl(int d, int bs, int g, const DecodeArgs& a, dim3 grid, int waves,
                        size_t lds, hipStream_t s) {
#define PA_DECODE_CASE(D_, BS_, G_)                                                       \
  if (d == D_ && bs == BS_ && g == G_) {                                                 \
    hipLaunchKernelGGL(                                                                  \
        (decode_kernel<ET, D_, BS_, G_, decode_prefetch(ET, D_, G_), true>),                 \
        grid, dim3(waves * 64), lds, s, a);                                              \
    return true;                                                                         \
  }
  PA_DECODE_SHAPES(PA_DECODE_CASE)
#undef PA_DECODE_CASE
  return false;
}

}  // namespace pa

namespace pa {

template <int ET>
int decode_groups_per_cu_impl(int d, int bs, int g, int waves, size_t lds) {
  int n = 0;
#define PA_OCC_CASE(D_, BS_, G_)                                                             \
  if (d == D_ && bs == BS_ && g == G_) {                                                    \
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(                                       \
            &n,                                                                             \
            decode_kernel<ET, D_, BS_, G_, decode_prefetch(ET, D_, G_), true>,                 \
            waves * 64, lds) != hipSuccess)                                                 \
      n = 0;                                                                                \
    return n;                                                                               \
  }
  PA_DECODE_SHAPES(PA_OCC_CASE)
#undef PA_OCC_CASE
  return 0;
}

}  // namespace pa
