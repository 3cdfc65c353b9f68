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
// * One workgroup of NW waves owns (sequence, KV head, partition).  Wave w of
//   the workgroup takes blocks w, w+NW, w+2NW, ... of the partition.
// * Rows are loaded in 16-byte chunks: lane = r*LPR + c holds chunk c of row r
//   of every RPI-row slab, so one load instruction covers RPI whole rows
//   (1 KiB, contiguous because the rows of a (block, head) pair are adjacent).
// * q.k: each lane dots its chunk against the same chunk of each query head
//   (bf16 pairs through v_dot2 with f32 accumulation), then the LPR lanes of a
//   row add up their partial sums with DPP row rotations; every lane of the
//   row ends with the identical score.
// * Running softmax per row group: lanes of row group r see only rows
//   r, r+RPI, ... of each tile, so each group keeps its own max m, weight sum
//   l and accumulator (for its D/LPR dims); no cross-row traffic happens
//   inside the loop.  Groups and waves are merged once at the end with the
//   log-sum-exp rule.
// * Scores are kept in log2 units, s*scale*log2(e), so the softmax weights are
//   exp2(s - m); the maximum itself gets exp2(0) = 1 exactly.
// * The block-table entries a wave needs are fetched with one vector load
//   (one entry per lane, up to 64 blocks) and handed out with v_readlane, so
//   each entry is read exactly once.
// * K/V tiles are double-buffered in registers: the loads of tile t+1 are in
//   flight while tile t is scored and accumulated.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

struct DecodeArgs {
  const uint8_t* q;
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* part_out;
  float* part_max;
  float* part_sum;
  int64_t num_blocks;
  int32_t num_kv_heads;
  int32_t num_heads;
  int32_t max_blocks;
  int32_t partition_blocks;  // blocks per partition; 0 = whole sequence
  int32_t max_parts;
  int32_t out_f32;           // 1: binary32 output; 0: bf16 output (bf16 cache only)
  float scale_log2;          // score scale * log2(e)
};

namespace dev {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// acc + q.k over one 16-byte chunk.
template <bool BF16>
__device__ __forceinline__ float dot16(float acc, const uint4& q, const uint4& k) {
  if constexpr (BF16) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.x),
                                         __builtin_bit_cast(bf16x2, q.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.y),
                                         __builtin_bit_cast(bf16x2, q.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.z),
                                         __builtin_bit_cast(bf16x2, q.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.w),
                                         __builtin_bit_cast(bf16x2, q.w), acc, false);
  } else {
    acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  }
  return acc;
}

// 16-byte chunk -> 8 (bf16) or 4 (f32) floats, exactly.
template <bool BF16>
__device__ __forceinline__ void unpack16(const uint4& c, float* v) {
  if constexpr (BF16) {
    v[0] = __uint_as_float(c.x << 16);
    v[1] = __uint_as_float(c.x & 0xFFFF0000u);
    v[2] = __uint_as_float(c.y << 16);
    v[3] = __uint_as_float(c.y & 0xFFFF0000u);
    v[4] = __uint_as_float(c.z << 16);
    v[5] = __uint_as_float(c.z & 0xFFFF0000u);
    v[6] = __uint_as_float(c.w << 16);
    v[7] = __uint_as_float(c.w & 0xFFFF0000u);
  } else {
    v[0] = __uint_as_float(c.x);
    v[1] = __uint_as_float(c.y);
    v[2] = __uint_as_float(c.z);
    v[3] = __uint_as_float(c.w);
  }
}

// binary32 -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

}  // namespace dev

template <bool BF16, int D, int BS, int G, int NW>
__global__ void __launch_bounds__(NW * 64) decode_kernel(DecodeArgs a) {
  using namespace dev;
  constexpr int EB = BF16 ? 2 : 4;                 // element bytes
  constexpr int VEC = 16 / EB;                     // elements per 16-byte chunk
  constexpr int LPR = D / VEC;                     // lanes per row
  constexpr int RPI = 64 / LPR;                    // rows per load instruction
  constexpr int TR = (BS < 4 * RPI) ? BS : 4 * RPI;  // rows per register tile
  constexpr int NI = TR / RPI;                     // load instructions per tile
  constexpr int TPB = BS / TR;                     // tiles per block
  static_assert(D % VEC == 0 && 64 % LPR == 0 && TR % RPI == 0 && BS % TR == 0, "tiling");
  static_assert(RPI * D * EB == 1024, "one load instruction covers 1 KiB");
  constexpr float NEG_INF = -__builtin_inff();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int r = lane / LPR;
  const int c = lane % LPR;

  int len = a.context_lens[seq];
  len = len < 0 ? 0 : (len > a.max_blocks * BS ? a.max_blocks * BS : len);
  const int nblk = (len + BS - 1) / BS;
  int blk_begin = 0;
  int blk_end = nblk;
  if (a.partition_blocks > 0) {
    blk_begin = part * a.partition_blocks;
    blk_end = min(nblk, blk_begin + a.partition_blocks);
    if (blk_begin >= blk_end) return;  // whole workgroup: no barrier skipped
  }

  const int head0 = kvh * G;
  const uint4* qrow =
      reinterpret_cast<const uint4*>(a.q + (size_t(seq) * a.num_heads + head0) * D * EB);
  uint4 qc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) qc[h] = qrow[h * LPR + c];

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = NEG_INF;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
  }

  const size_t head_bytes = size_t(BS) * D * EB;
  const size_t block_bytes = head_bytes * a.num_kv_heads;
  const uint8_t* kbase = a.k_pool + kvh * head_bytes;
  const uint8_t* vbase = a.v_pool + kvh * head_bytes;
  const int32_t* trow = a.block_tables + size_t(seq) * a.max_blocks;
  const float cl2 = a.scale_log2;

  const int span = blk_end - blk_begin;
  const int nmine = span > wave ? (span - wave + NW - 1) / NW : 0;

  for (int k0 = 0; k0 < nmine; k0 += 64) {
    const int kk = min(64, nmine - k0);
    int tbl = -1;
    if (lane < kk) {
      const int e = trow[blk_begin + wave + (k0 + lane) * NW];
      tbl = (e >= 0 && int64_t(e) < a.num_blocks) ? e : -1;
    }
    const int ntiles = kk * TPB;

    auto load = [&](uint4(&kr)[NI], uint4(&vr)[NI], int t) {
      const int phys = __builtin_amdgcn_readlane(tbl, t / TPB);
      if (phys < 0) return;
      const size_t off = size_t(phys) * block_bytes + size_t(t % TPB) * (TR * D * EB);
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + off) + lane;
      const uint4* vp = reinterpret_cast<const uint4*>(vbase + off) + lane;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        kr[i] = kp[i * 64];
        vr[i] = vp[i * 64];
      }
    };

    auto process = [&](const uint4(&kr)[NI], const uint4(&vr)[NI], int t) {
      const int phys = __builtin_amdgcn_readlane(tbl, t / TPB);
      const int tok0 = (blk_begin + wave + (k0 + t / TPB) * NW) * BS + (t % TPB) * TR;
      const int nvalid = phys < 0 ? 0 : min(TR, len - tok0);
      if (nvalid <= 0) return;
      float s[NI][G];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h)
          s[i][h] = group_sum<LPR>(dot16<BF16>(0.f, qc[h], kr[i])) * cl2;
      const bool partial = nvalid < TR;
      if (partial) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
          if (i * RPI + r >= nvalid)
#pragma unroll
            for (int h = 0; h < G; ++h) s[i][h] = NEG_INF;
      }
      float p[NI][G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = s[0][h];
#pragma unroll
        for (int i = 1; i < NI; ++i) mx = fmaxf(mx, s[i][h]);
        const float mnew = fmaxf(m[h], mx);
        const float base = (mnew == NEG_INF) ? 0.f : mnew;
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
        unpack16<BF16>(vr[i], v);
        if (partial && i * RPI + r >= nvalid) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = 0.f;  // masked rows may hold NaN
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(p[i][h], v[e], acc[h][e]);
      }
    };

    uint4 ka[NI], va[NI], kb[NI], vb[NI];
    load(ka, va, 0);
    for (int t = 0; t < ntiles; t += 2) {
      if (t + 1 < ntiles) load(kb, vb, t + 1);
      process(ka, va, t);
      if (t + 1 < ntiles) {
        if (t + 2 < ntiles) load(ka, va, t + 2);
        process(kb, vb, t + 1);
      }
    }
  }

  // Merge the RPI row groups of this wave (lanes that differ in r).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float big = m[h];
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) big = fmaxf(big, __shfl_xor(big, off));
    const float f = (m[h] == NEG_INF) ? 0.f : fast_exp2(m[h] - big);
    float lw = l[h] * f;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) lw += __shfl_xor(lw, off);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float x = acc[h][e] * f;
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off);
      acc[h][e] = x;
    }
    m[h] = big;
    l[h] = lw;
  }

  // Merge the NW waves through LDS and write the result.
  __shared__ float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_acc[wave][h][c * VEC + e] = acc[h][e];
      if (c == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < G * D; o += NW * 64) {
    const int h = o / D;
    const int d = o - h * D;
    float big = NEG_INF;
#pragma unroll
    for (int w = 0; w < NW; ++w) big = fmaxf(big, s_m[w][h]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_m[w][h];
      const float f = (mw == NEG_INF) ? 0.f : fast_exp2(mw - big);
      lsum = fmaf(f, s_l[w][h], lsum);
      osum = fmaf(f, s_acc[w][h][d], osum);
    }
    const float val = lsum > 0.f ? osum / lsum : 0.f;
    const int head = head0 + h;
    if (a.partition_blocks > 0) {
      const size_t row = (size_t(seq) * a.num_heads + head) * a.max_parts + part;
      a.part_out[row * D + d] = val;
      if (d == 0) {
        a.part_max[row] = big == NEG_INF ? NEG_INF : big * 0.69314718055994531f;  // ln 2
        a.part_sum[row] = lsum;
      }
    } else {
      const size_t idx = (size_t(seq) * a.num_heads + head) * D + d;
      if (BF16 && !a.out_f32)
        static_cast<uint16_t*>(a.out)[idx] = to_bf16(val);
      else
        static_cast<float*>(a.out)[idx] = val;
    }
  }
}

// Launches decode_kernel<BF16, D, BS, G, 4> for a runtime (D, BS, G);
// returns false when no instantiation matches.
bool launch_decode_f32(int d, int bs, int g, const DecodeArgs& a, dim3 grid, hipStream_t s);
bool launch_decode_bf16(int d, int bs, int g, const DecodeArgs& a, dim3 grid, hipStream_t s);

constexpr int kDecodeWaves = 4;

}  // namespace pa

namespace pa {

// Instantiation table: D in {64, 128}, block size in {16, 32}, G in {1, 2, 4, 8}.
template <bool BF16>
bool launch_decode_impl(int d, int bs, int g, const DecodeArgs& a, dim3 grid, hipStream_t s) {
#define PA_DECODE_CASE(D_, BS_, G_)                                                     \
  if (d == D_ && bs == BS_ && g == G_) {                                               \
    hipLaunchKernelGGL((decode_kernel<BF16, D_, BS_, G_, kDecodeWaves>), grid,         \
                       dim3(kDecodeWaves * 64), 0, s, a);                              \
    return true;                                                                       \
  }
#define PA_DECODE_G(D_, BS_) \
  PA_DECODE_CASE(D_, BS_, 1) PA_DECODE_CASE(D_, BS_, 2) PA_DECODE_CASE(D_, BS_, 4) PA_DECODE_CASE(D_, BS_, 8)
  PA_DECODE_G(64, 16)
  PA_DECODE_G(64, 32)
  PA_DECODE_G(128, 16)
  PA_DECODE_G(128, 32)
#undef PA_DECODE_G
#undef PA_DECODE_CASE
  return false;
}

}  // namespace pa
