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
//   never synchronise after the preamble; each owns its head end to end.
// * Work unit = one (sequence, block).  Three ways to hand units out:
//   single pass (a workgroup per sequence), fixed partitions (a workgroup per
//   (sequence, partition), writing split-KV partials), and balanced (a fixed
//   grid; all units of the batch are split evenly over the workgroups, so a
//   workgroup's range holds whole sequences and pieces of sequences; whole
//   ones write the output, pieces write partials merged by merge_kernel).
// * Rows are loaded in 16-byte chunks with non-temporal loads (the cache is
//   streamed once): lane = r*LPR + c holds chunk c of rows r, r+RPI, ..., so
//   one load instruction covers RPI whole rows (1 KiB contiguous).
// * q.k: each lane dots its chunk against the same chunk of each query head
//   (bf16 pairs through v_dot2 with f32 accumulation), then the LPR lanes of a
//   row add up their partial sums with DPP row rotations; every lane of the
//   row ends with the identical score.
// * Running softmax per row group (lanes with equal r see rows r, r+RPI, ...):
//   no cross-row traffic inside the loop; row groups are merged once per
//   piece with the log-sum-exp rule.  Scores are kept in log2 units
//   (s*scale*log2 e), so weights are exp2(s - m) and the maximum gets exactly 1.
// * Block-table entries of up to 64 units are fetched with one vector load
//   (one per lane) and handed out with v_readlane, so each is read once.
// * K/V tiles sit in a ring of PF+1 register buffers: the loads of the next
//   PF tiles are in flight while the current tile is scored and accumulated,
//   across sequence boundaries too.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

enum DecodeMode : int32_t { kModeSingle = 0, kModePartition = 1, kModeBalanced = 2 };

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
  int32_t* info;        // balanced: [0] total units, [1 + i] first unit of sequence i (i <= S)
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t num_heads;
  int32_t max_blocks;
  int32_t mode;
  int32_t partition_blocks;  // partition mode: blocks per partition
  int32_t max_parts;         // partition mode: partitions per (sequence, head) row
  int32_t num_groups;        // balanced mode: workgroups sharing the units
  int32_t out_f32;           // 1: binary32 output; 0: bf16 output (bf16 cache only)
  float scale_log2;          // score scale * log2(e)
};

struct MergeArgs {
  const float* piece_out;
  const float* piece_max;
  const float* piece_sum;
  const int32_t* info;
  void* out;
  int32_t num_heads;
  int32_t num_groups;
  int32_t out_f32;
};

namespace dev {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
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

// 16-byte chunk -> 8 (bf16) or 4 (f32) floats, exactly.
template <bool BF16>
__device__ __forceinline__ void unpack16(const u32x4& c, float* v) {
  if constexpr (BF16) {
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

// binary32 -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Workgroup that processes unit u when `total` units are split evenly over
// `groups` workgroups (workgroup g takes [g*total/groups, (g+1)*total/groups)).
__device__ __forceinline__ int group_of_unit(int64_t u, int64_t total, int64_t groups) {
  return int(((u + 1) * groups + total - 1) / total - 1);
}

}  // namespace dev

template <bool BF16, int D, int BS, int G, int PF, bool NT>
__global__ void __launch_bounds__(512) decode_kernel(DecodeArgs a) {
  using namespace dev;
  constexpr int EB = BF16 ? 2 : 4;                   // element bytes
  constexpr int VEC = 16 / EB;                       // elements per 16-byte chunk
  constexpr int LPR = D / VEC;                       // lanes per row
  constexpr int RPI = 64 / LPR;                      // rows per load instruction
  constexpr int TRW = (G >= 8 ? 2 : 4) * RPI;        // wide groups keep smaller tiles
  constexpr int TR = BS < TRW ? BS : TRW;            // rows per register tile
  constexpr int NI = TR / RPI;                       // load instructions per tile
  constexpr int TPB = BS / TR;                       // tiles per block
  constexpr int NB = PF + 1;                         // ring buffers
  constexpr bool QPF = G <= 4;                       // prefetch the next piece's query
  static_assert(D % VEC == 0 && 64 % LPR == 0 && TR % RPI == 0 && BS % TR == 0, "tiling");
  static_assert(RPI * D * EB == 1024, "one load instruction covers 1 KiB");

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
  int fixed_seq = -1;
  int64_t ubeg, uend;
  if (a.mode == kModeBalanced) {
    const int S = a.num_seqs;
    for (int i = threadIdx.x; i < S; i += blockDim.x) {
      int len = a.context_lens[i];
      len = len < 0 ? 0 : (len > max_tokens ? max_tokens : len);
      s_prefix[i + 1] = (len + BS - 1) / BS;
    }
    if (threadIdx.x == 0) s_prefix[0] = 0;
    __syncthreads();
    if (wave == 0) {
      int carry = 0;
      for (int base = 0; base < S; base += 64) {
        const int i = base + lane;
        int v = i < S ? s_prefix[i + 1] : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int up = __shfl_up(v, off);
          if (lane >= off) v += up;
        }
        if (i < S) s_prefix[i + 1] = carry + v;
        carry += __shfl(v, 63);
      }
    }
    __syncthreads();
    const int64_t total_units = s_prefix[S];
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      for (int i = threadIdx.x; i <= S; i += blockDim.x) a.info[1 + i] = s_prefix[i];
      if (threadIdx.x == 0) a.info[0] = int32_t(total_units);
    }
    ubeg = int64_t(blockIdx.x) * total_units / a.num_groups;
    uend = int64_t(blockIdx.x + 1) * total_units / a.num_groups;
  } else {
    fixed_seq = a.mode == kModeSingle ? blockIdx.x : blockIdx.z;
    int len = a.context_lens[fixed_seq];
    len = len < 0 ? 0 : (len > max_tokens ? max_tokens : len);
    const int nblk = (len + BS - 1) / BS;
    ubeg = 0;
    uend = nblk;
    if (a.mode == kModePartition) {
      ubeg = int64_t(blockIdx.x) * a.partition_blocks;
      uend = min(int64_t(nblk), ubeg + a.partition_blocks);
      if (ubeg >= uend) return;  // whole workgroup, before any barrier
    }
  }

  const size_t head_bytes = size_t(BS) * D * EB;
  const size_t block_bytes = head_bytes * a.num_kv_heads;
  const uint8_t* kbase = a.k_pool + kvh * head_bytes;
  const uint8_t* vbase = a.v_pool + kvh * head_bytes;
  const float cl2 = a.scale_log2;

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
  float m[G], l[G], acc[G][VEC];
  auto reset = [&]() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
    }
  };
  reset();
  u32x4 qc[G], qn[QPF ? G : 1];
  auto load_q = [&](u32x4(&dst)[G], int seq) {
    const u32x4* qrow = reinterpret_cast<const u32x4*>(
        a.q + (size_t(seq) * a.num_heads + head0) * D * EB);
#pragma unroll
    for (int h = 0; h < G; ++h) dst[h] = qrow[h * LPR + c];
  };

  // Emit the finished piece (blocks j_first..j_last) of sequence `seq`.
  auto emit = [&](int seq, int j_first, int j_last, int len) {
    // merge the RPI row groups (lanes that differ in r)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float big = m[h];
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) big = fmaxf(big, __shfl_xor(big, off));
      const float f = (m[h] == kNegInf) ? 0.f : fast_exp2(m[h] - big);
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
    if (r != 0) return;
    const int nblk = (len + BS - 1) / BS;
    const bool whole = a.mode == kModeSingle ||
                       (a.mode == kModeBalanced && j_first == 0 && j_last == nblk - 1);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
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

  // ---- chunks of up to 64 units ------------------------------------------------
  // A piece may run on into the next chunk (same sequence): then its state,
  // query and first block carry over.
  bool carry = false;
  int cur_seq = 0, cur_first = 0;
  for (int64_t c0 = ubeg; c0 < uend; c0 += 64) {
    const int n = int(min(int64_t(64), uend - c0));
    // per-lane unit description: sequence, block index, context length, physical block
    int sk = 0, jk = 0, lk = 0, pk = -1;
    if (lane < n) {
      const int64_t u = c0 + lane;
      if (fixed_seq >= 0) {
        sk = fixed_seq;
        jk = int(u);
      } else {
        int lo = 0, hi = a.num_seqs;  // s_prefix[lo] <= u < s_prefix[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_prefix[mid] <= u) lo = mid; else hi = mid;
        }
        sk = lo;
        jk = int(u - s_prefix[lo]);
      }
      const int len = a.context_lens[sk];
      lk = len < 0 ? 0 : (len > max_tokens ? max_tokens : len);
      const int e = a.block_tables[size_t(sk) * a.max_blocks + jk];
      pk = (e >= 0 && int64_t(e) < a.num_blocks) ? e : -1;
    }
    // piece starts: units whose sequence differs from the previous unit's
    const int sprev = __shfl_up(sk, 1);
    const uint64_t starts = __ballot(lane < n && (lane == 0 ? !carry : sk != sprev));
    // does the piece open at the chunk's end continue into the next chunk?
    const int last_seq = __builtin_amdgcn_readlane(sk, n - 1);
    const bool cont = c0 + n < uend && (fixed_seq >= 0 || c0 + n < s_prefix[last_seq + 1]);

    if (!carry) {
      cur_seq = __builtin_amdgcn_readlane(sk, 0);
      cur_first = __builtin_amdgcn_readlane(jk, 0);
      load_q(qc, cur_seq);
    }
    uint64_t later = starts & ~uint64_t(1);  // piece starts after the current piece
    if constexpr (QPF)
      if (later) load_q(qn, __builtin_amdgcn_readlane(sk, __builtin_ctzll(later)));

    auto load_tile = [&](u32x4(&kr)[NI], u32x4(&vr)[NI], int t) {
      const int phys = __builtin_amdgcn_readlane(pk, t / TPB);
      if (phys < 0) return;
      const size_t off = size_t(phys) * block_bytes + size_t(t % TPB) * (TR * D * EB);
      const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + off) + lane;
      const u32x4* vp = reinterpret_cast<const u32x4*>(vbase + off) + lane;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        kr[i] = load16<NT>(kp + i * 64);
        vr[i] = load16<NT>(vp + i * 64);
      }
    };

    auto process_tile = [&](const u32x4(&kr)[NI], const u32x4(&vr)[NI], int t) {
      const int ut = t / TPB;
      const int sub = t % TPB;
      if (sub == 0 && ut > 0 && ((starts >> ut) & 1)) {
        // a new piece begins (its query was prefetched into qn when QPF)
        cur_seq = __builtin_amdgcn_readlane(sk, ut);
        cur_first = __builtin_amdgcn_readlane(jk, ut);
        if constexpr (QPF) {
#pragma unroll
          for (int h = 0; h < G; ++h) qc[h] = qn[h];
          later &= ~((uint64_t(2) << ut) - 1);
          if (later) load_q(qn, __builtin_amdgcn_readlane(sk, __builtin_ctzll(later)));
        } else {
          load_q(qc, cur_seq);
        }
      }
      const int phys = __builtin_amdgcn_readlane(pk, ut);
      const int j = __builtin_amdgcn_readlane(jk, ut);
      const int len = __builtin_amdgcn_readlane(lk, ut);
      const int tok0 = j * BS + sub * TR;
      const int nvalid = phys < 0 ? 0 : min(TR, len - tok0);
      if (nvalid > 0) {
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
      }
      const bool piece_end =
          sub == TPB - 1 && (ut == n - 1 ? !cont : ((starts >> (ut + 1)) & 1));
      if (piece_end) {
        emit(cur_seq, cur_first, j, len);
        reset();
      }
    };

    const int ntiles = n * TPB;
    u32x4 kb[NB][NI], vb[NB][NI];
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (i < ntiles) load_tile(kb[i], vb[i], i);
    for (int t0 = 0; t0 < ntiles; t0 += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int t = t0 + u;
        if (t < ntiles) {
          if (t + PF < ntiles) load_tile(kb[(u + PF) % NB], vb[(u + PF) % NB], t + PF);
          process_tile(kb[u], vb[u], t);
        }
      }
    }
    carry = cont;
  }
}

// Merge the pieces of each sequence that more than one workgroup worked on
// (balanced mode), and write zeros for empty sequences.  One wave per
// (sequence, query head); pieces carry log2-unit maxima.
template <int D>
__global__ void __launch_bounds__(64) merge_kernel(MergeArgs a) {
  using namespace dev;
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const int head = blockIdx.x;
  const int seq = blockIdx.y;
  const int64_t total = a.info[0];
  const int64_t u0 = a.info[1 + seq];
  const int64_t u1 = a.info[2 + seq];  // one past the sequence's last unit
  const size_t orow = (size_t(seq) * a.num_heads + head) * D;
  float accv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) accv[e] = 0.f;
  float wsum = 0.f;
  if (u1 > u0) {
    const int g0 = group_of_unit(u0, total, a.num_groups);
    const int g1 = group_of_unit(u1 - 1, total, a.num_groups);
    if (g0 == g1) return;  // one workgroup held the whole sequence and wrote it
    float big = kNegInf;
    for (int g = g0; g <= g1; ++g) {
      const size_t row = (size_t(g) + seq) * a.num_heads + head;
      if (a.piece_sum[row] > 0.f) big = fmaxf(big, a.piece_max[row]);
    }
    for (int g = g0; g <= g1; ++g) {
      const size_t row = (size_t(g) + seq) * a.num_heads + head;
      const float s = a.piece_sum[row];
      if (!(s > 0.f)) continue;
      const float w = s * fast_exp2(a.piece_max[row] - big);
      wsum += w;
#pragma unroll
      for (int e = 0; e < PER; ++e)
        accv[e] = fmaf(w, a.piece_out[row * D + e * 64 + lane], accv[e]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float val = accv[e] * inv;
    if (a.out_f32)
      static_cast<float*>(a.out)[orow + e * 64 + lane] = val;
    else
      static_cast<uint16_t*>(a.out)[orow + e * 64 + lane] = uint16_t(to_bf16(val));
  }
}

// Launches decode_kernel for a runtime (D, BS, G) on a grid of `waves`-wave
// workgroups with `lds` bytes of dynamic LDS; false when no instantiation matches.
bool launch_decode_f32(int d, int bs, int g, const DecodeArgs& a, dim3 grid, int waves,
                       size_t lds, hipStream_t s);
bool launch_decode_bf16(int d, int bs, int g, const DecodeArgs& a, dim3 grid, int waves,
                        size_t lds, hipStream_t s);

// Instantiation table: D in {64, 128}, block size in {16, 32}, G in {1, 2, 4, 8}.
template <bool BF16>
bool launch_decode_impl(int d, int bs, int g, const DecodeArgs& a, dim3 grid, int waves,
                        size_t lds, hipStream_t s) {
#define PA_DECODE_CASE(D_, BS_, G_)                                                       \
  if (d == D_ && bs == BS_ && g == G_) {                                                 \
    hipLaunchKernelGGL((decode_kernel<BF16, D_, BS_, G_, (G_ <= 4 ? 2 : 1), true>), grid, \
                       dim3(waves * 64), lds, s, a);                                     \
    return true;                                                                         \
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
