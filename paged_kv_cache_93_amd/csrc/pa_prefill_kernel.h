// Mixed-batch (prefill) attention over the paged cache, for gfx950.
//
// What it computes ("How Paged Attention and Continuous Batching Actually
// Work", section "Continuous batching: schedule steps, not batches": every
// scheduled token of the batch flattened into one sequence, metadata saying
// where each request's tokens begin and end and what they may see;
// "PagedAttention and continuous batching", section "Attention kernel
// modification": causal attention of position t over K_{0:t}, V_{0:t} loaded
// block by block through the table, with a running softmax): sequence i owns
// query rows query_start[i] .. query_start[i+1]-1, its n_i tokens are its last
// n_i positions, and token j at position p = L_i - n_i + j attends to
// positions 0..p.  A decode row is n_i = 1.
//
// Mapping onto CDNA4:
// * A workgroup (4 waves) takes a tile of 128 query rows of one sequence and
//   one KV head: floor(128/G) tokens times the G query heads that share the
//   KV head (rows past those tokens are idle), so every K/V row the tile
//   loads serves all of them.  Each wave owns 32 rows (two 16-row MFMA tiles).
// * The tile walks its keys 32 at a time (positions 0 .. its last row's
//   position).  The workgroup stages each 32-key K/V tile in LDS, row-major
//   with XOR-swizzled 16-byte pieces: the MFMA A operand of S^T = K Q^T reads
//   16-byte K row pieces, and the A operand of O^T = V^T P^T (keys contiguous
//   per dimension) comes from the transposed LDS read.  Tiles go in by LDS
//   DMA; 8-bit codes land as they are in the half of the stage that rows
//   16..31 take and the workgroup expands them into the bf16 layout in LDS
//   (exact; the scales are folded into the score scale and the output).  A
//   register-staged kernel, which converts the codes on their way from
//   memory, stays as the comparison path (PA_PREFILL_DMA / _DMA_FP8 = 0).
// * Scores come out as S^T, so lane 16g + r holds keys 4g..4g+3 (and 16 +
//   4g..) of query row r: the softmax weights P are already the B operand of
//   O^T = V^T P^T in that lane (the k order of the two operands is permuted
//   alike), and the output O^T lands in the lane that owns the row's running
//   max and sum - no shuffles except two lane swaps for the row maximum.
// * For a bf16 output, weights are rounded to bf16 for the matrix product, and
//   the running sum adds the rounded weights, so the output is an exact convex
//   combination of V rows; each weight is rounded to nearest even (within 2^-8
//   of its value, relative), so after the normalisation the weights are within
//   about 2^-7.  For a float32 output each weight enters the product as three
//   bf16 terms (within 2^-24 of it) and the sum adds the float32 weights.
#pragma once

#include <type_traits>

#include "pa_decode_kernel.h"
#include "pa_internal.h"

namespace pa {
namespace pf {

using namespace dev;

constexpr int kD = 128;           // head dim
constexpr int kRows = 128;        // query rows per workgroup tile
constexpr int kWaves = 4;
constexpr int kKeys = 32;         // keys per K/V tile
// The register-staged kernel's K and V tiles in LDS: bf16 rows of 256 bytes
// with the bf16 ring's piece swizzles
constexpr int kKBytes = kKeys * kD * 2;
constexpr int kVBytes = kKeys * kD * 2;
constexpr int kBufBytes = kKBytes + kVBytes;
// Block-table entries a workgroup keeps in LDS behind its tile buffers: a
// window of the walk's blocks, reloaded when the walk passes its end.  (Vector
// memory operations complete in order, so an entry loaded from global memory
// inside the walk would wait for every tile load issued before it.)
constexpr int kTblWin = 1024;

#ifndef PA_PREFILL_ROW_TILES
#define PA_PREFILL_ROW_TILES 2  // 16-row tiles per wave of the LDS-DMA kernel: 2 or 4
#endif

#ifndef PA_PREFILL_DMA
#define PA_PREFILL_DMA 1  // 0: bf16 caches take the register-staged kernel too (for comparison)
#endif
#ifndef PA_PREFILL_DMA_FP8
#define PA_PREFILL_DMA_FP8 1  // 0: 8-bit caches take the register-staged kernel
#endif

#ifndef PA_PREFILL_KSWZ
#define PA_PREFILL_KSWZ 16  // K rows whose pieces the swizzle spreads (16; 8 for comparison)
#endif
#ifndef PA_PREFILL_VSWZ
#define PA_PREFILL_VSWZ 8   // V rows whose piece pairs the swizzle spreads (8; 4 for comparison)
#endif

typedef short v4s __attribute__((ext_vector_type(4)));
#define PA_LDS(T) __attribute__((address_space(3))) T

constexpr bf16x2 kOnes = {__bf16(1.0f), __bf16(1.0f)};

struct PrefillArgs {
  const uint8_t* q;
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* block_tables;
  const int32_t* query_start;
  const int32_t* context_lens;
  const int32_t* tiles;  // [0] tile count; then (sequence, tile index) pairs
  void* out;
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t num_heads;
  int32_t max_blocks;
  int32_t max_tiles;
  float scale_log2;  // score scale * log2(e), times the K pool's scale (8-bit cache)
  float v_scale;     // the V pool's scale (8-bit cache), else 1
  const float* k_scales;  // 8-bit cache with one scale per KV head (then the two above
  const float* v_scales;  //   leave them out), or NULL
  int32_t window;    // sliding window in tokens (0: none)
  const float* alibi;  // ALiBi slope per query head, or NULL
};

// One 32-key tile of the online softmax for a wave's two 16-row tiles: scores
// (S^T in the MFMA C layout: lane 16g + r holds keys 4g..4g+3 and 16+4g..
// 16+4g+3 of row r) -> masked, exponentiated weights packed as the B operand
// of O^T = V^T P^T in the k order [4g .. 4g+3, 16+4g .. 16+4g+3]; the running
// max, sum and accumulators of the rows are updated.  Only tiles that reach
// past the workgroup's first position (or, with a window, start before its
// last row's window) need masks; without ALiBi the max is taken on raw
// scores (the scale is positive) and the scale enters with the exponent's fma.
//
// PT: bf16 terms per weight.  With one, each weight is rounded to bf16 and
// the running sum adds the rounded weights (the output is an exact convex
// combination of V rows with weights within about 2^-7 of the true ones).
// With three (float32 outputs), weight p goes in as hi + mid + lo, hi its
// bf16 rounding, mid that of p - hi, lo that of the rest (both differences
// exact in float32), which leaves p within 2^-24 of its value; the running
// sum adds the float32 weights.  pf[t][rt] is term t.
template <bool AL, int NR = 2, int PT = 1>
__device__ __forceinline__ void softmax_step(f32x4 (&s)[NR][2], u32x4 (&pf)[PT][NR], int k0,
                                             const int (&pos)[NR], const int (&lo_row)[NR],
                                             const float (&slope2)[NR], int min_pos, int max_pos,
                                             int W, float sc, int grp, float (&m)[NR],
                                             float (&lsum)[NR], f32x4 (&acc)[NR][8]) {
  static_assert(PT == 1 || PT == 3, "one or three bf16 terms per weight");
  if constexpr (AL) {
    // scores to log2 units plus slope * (key - position)
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
      const float sd = slope2[rt] * float(k0 + 4 * grp - pos[rt]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          s[rt][h][v] = fmaf(s[rt][h][v], sc, fmaf(slope2[rt], float(16 * h + v), sd));
    }
  }
  if (k0 + kKeys - 1 > min_pos || (W > 0 && k0 < max_pos - W + 1)) {
#pragma unroll
    for (int rt = 0; rt < NR; ++rt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int k = k0 + 16 * h + 4 * grp + v;
          if (k > pos[rt] || k < lo_row[rt]) s[rt][h][v] = kNegInf;
        }
  }
  // The exponent base moves only when the row maximum passes it by more than 8
  // (log2 units): weights stay <= 2^8, the accumulators are rescaled rarely,
  // and the result is the same softmax.  A row's maximum passes its base only
  // if one of its four lanes' maxima does, so the lanes test their own maxima
  // first and the row maxima (two lane swaps each) and the new bases are
  // taken only when some row of the wave moves.
  float lmx[NR], base[NR], alpha[NR];
  bool up = false;
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) {
    lmx[rt] = fmaxf(fmaxf(fmaxf(s[rt][0][0], s[rt][0][1]), fmaxf(s[rt][0][2], s[rt][0][3])),
                    fmaxf(fmaxf(s[rt][1][0], s[rt][1][1]), fmaxf(s[rt][1][2], s[rt][1][3])));
    up |= (AL ? lmx[rt] : lmx[rt] * sc) > m[rt] + 8.f;
    base[rt] = m[rt] == kNegInf ? 0.f : m[rt];
    alpha[rt] = 1.f;
  }
  bool moved[NR] = {};
  if (__ballot(up) != 0) {
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
      float mx = xor_max<16>(lmx[rt]);
      if constexpr (!AL) mx *= sc;
      const bool move = mx > m[rt] + 8.f;
      const float mnew = move ? mx : m[rt];
      base[rt] = mnew == kNegInf ? 0.f : mnew;
      alpha[rt] = move ? fast_exp2(m[rt] - base[rt]) : 1.f;
      m[rt] = mnew;
      moved[rt] = __ballot(move) != 0;
    }
  }
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) {
    float psum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int h = w >> 1, v = 2 * (w & 1);
      f32x2 pp;
      if constexpr (AL)
        pp = f32x2{fast_exp2(s[rt][h][v] - base[rt]), fast_exp2(s[rt][h][v + 1] - base[rt])};
      else
        pp = f32x2{fast_exp2(fmaf(s[rt][h][v], sc, -base[rt])),
                   fast_exp2(fmaf(s[rt][h][v + 1], sc, -base[rt]))};
      const bf16x2 pb = __builtin_convertvector(pp, bf16x2);
      pf[0][rt][w] = __builtin_bit_cast(uint32_t, pb);
      if constexpr (PT == 1) {
        psum = __builtin_amdgcn_fdot2_f32_bf16(pb, kOnes, psum, false);  // adds the rounded pair
      } else {
        const f32x2 r1 = pp - __builtin_convertvector(pb, f32x2);
        const bf16x2 pm = __builtin_convertvector(r1, bf16x2);
        const f32x2 r2 = r1 - __builtin_convertvector(pm, f32x2);
        pf[1][rt][w] = __builtin_bit_cast(uint32_t, pm);
        pf[2][rt][w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2));
        psum += pp[0] + pp[1];
      }
    }
    lsum[rt] = fmaf(lsum[rt], alpha[rt], psum);
    if (moved[rt]) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[rt][dt] *= alpha[rt];
    }
  }
}

template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  // s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding; expcnt left at its maximum)
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

template <int ET, int BS, int G, bool OUT_F32, bool AL>
__global__ void __launch_bounds__(256, 2) prefill_kernel(PrefillArgs a) {
  constexpr int EB = ET == kFP8 ? 1 : 2;   // K/V element bytes
  constexpr int TT = kRows / G;            // tokens per tile
  using Raw = typename LaneChunk<8 * EB>::type;  // 8 elements of a row
  extern __shared__ __attribute__((aligned(16))) uint8_t s_mem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups go to the 8 XCDs round-robin by linear id; renumber them so
  // each XCD takes a contiguous run of (KV head, tile) items - the tiles of one
  // sequence and head then share that XCD's L2.
  const int nwg = gridDim.x * gridDim.y;
  const int id = blockIdx.y * gridDim.x + blockIdx.x;
  const int xcd = id % 8, slot = id / 8;
  const int logical = xcd * (nwg / 8) + min(xcd, nwg % 8) + slot;
  const int t = logical % gridDim.x;
  const int g = logical / gridDim.x;
  const float sl2 = a.k_scales ? a.scale_log2 * a.k_scales[g] : a.scale_log2;
  const float vsc = a.v_scales ? a.v_scales[g] : a.v_scale;
  if (t >= a.tiles[0]) return;
  const int seq = a.tiles[1 + 2 * t];
  const int tile = a.tiles[2 + 2 * t];
  if (seq < 0 || seq >= a.num_seqs) return;

  const int32_t qs0 = min(max(a.query_start[seq], 0), a.num_tokens);
  const int32_t qs1 = min(max(a.query_start[seq + 1], 0), a.num_tokens);
  const int32_t n = qs1 - qs0;
  const int32_t max_len = a.max_blocks * BS;
  const int32_t L = min(max(a.context_lens[seq], 0), max_len);
  const int32_t c = L - n;  // position of query token 0 (negative: caller error)
  const int32_t j0 = tile * TT;
  const int32_t j1 = min(j0 + TT, n);
  if (j1 <= j0) return;
  const int32_t kend = c + j1;  // keys 0 .. kend-1 are needed (kend <= L)
  const int32_t* table = a.block_tables + int64_t(seq) * a.max_blocks;

  // ---- this lane's query rows and their fragments (B operand of S^T) --------
  const int r16 = lane & 15, grp = lane >> 4;
  int pos[2];
  bool valid[2];
  int64_t row_index[2];  // output row (token * Hq + head)
  u32x4 qf[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = wave * 32 + rt * 16 + r16;
    const int tok = j0 + row / G;
    valid[rt] = tok < j1;
    const int tq = min(tok, j1 - 1);
    pos[rt] = c + tok;
    const int head = g * G + row % G;
    row_index[rt] = int64_t(qs0 + tq) * a.num_heads + head;
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + row_index[rt] * kD * 2);
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) qf[rt][mm] = qp[4 * mm + grp];
  }

  // ---- K/V tile staging -------------------------------------------------------
  // Thread tid loads dims [8*dc, 8*dc+8) of keys 2kp and 2kp+1 of a tile (one
  // block: block sizes are even), into its register pair e = 0, 1 as keys
  // 2kp + (e ^ par), par = kp % 2: a 16-byte LDS store of register e then
  // writes rows of both parities in each half-wave (rows 256 bytes apart fall
  // in different bank halves), where keys in order would put two rows of one
  // parity on the same banks.  Loads run two tiles ahead of the math (two
  // register sets).  Every walk step issues the same four loads, so the
  // compiler's wait before a register set is stored counts exactly the loads
  // issued after it: keys past the context and blocks outside the pool read
  // block 0 of the pool instead, and a per-set mask zeroes those rows when the
  // set is stored.
  const int dc = tid & 15, kp = tid >> 4, par = kp & 1;
  Raw kr[2][2], vr[2][2];
  int zmask[2] = {0, 0};  // bit e: key 2kp + (e ^ par) of the set's tile reads as zero
  // key 2kp of a tile sits at row (2kp) % BS of its block (tiles start at
  // multiples of 32, a multiple of BS), so a lane's offset inside a block is fixed
  constexpr int kRowBytes = kD * EB;
  const int64_t blk_stride = int64_t(a.num_kv_heads) * BS * kRowBytes;
  const int64_t lane_off = (int64_t(g) * BS + (2 * kp) % BS) * kRowBytes + dc * 8 * EB;

  // the walk's table entries, a window of kTblWin of them in LDS (entries
  // outside the pool stored as -1)
  int32_t* s_tbl = reinterpret_cast<int32_t*>(s_mem + 2 * kBufBytes);
  const int nblk = kend > 0 ? (kend + BS - 1) / BS : 0;
  int tbl0 = 0;  // first block the window holds
  auto load_tbl = [&](int first) {
    tbl0 = first;
    const int cnt = min(kTblWin, nblk - first);
    for (int i = tid; i < cnt; i += 256) {
      const int p = table[first + i];
      s_tbl[i] = (p < 0 || int64_t(p) >= a.num_blocks) ? -1 : p;
    }
  };
  auto load_tile = [&](int set, int k0) {
    const int key = k0 + 2 * kp;  // and key + 1, in the same block
    const int phys = key < kend ? s_tbl[key / BS - tbl0] : -1;
    zmask[set] = phys < 0 ? 3 : (key + 1 < kend ? 0 : (par ? 1 : 2));
    const int64_t off = int64_t(phys < 0 ? 0 : phys) * blk_stride + lane_off;
    const int64_t o0 = off + par * kRowBytes, o1 = off + (par ^ 1) * kRowBytes;
    kr[set][0] = *reinterpret_cast<const Raw*>(a.k_pool + o0);
    kr[set][1] = *reinterpret_cast<const Raw*>(a.k_pool + o1);
    vr[set][0] = *reinterpret_cast<const Raw*>(a.v_pool + o0);
    vr[set][1] = *reinterpret_cast<const Raw*>(a.v_pool + o1);
  };
  auto store_tile = [&](int set, int buf) {
    u32x4* lk = reinterpret_cast<u32x4*>(s_mem + buf * kBufBytes);
    uint8_t* lv = s_mem + buf * kBufBytes + kKBytes;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 2 * kp + (e ^ par);
      const bool z = (zmask[set] >> e) & 1;
      const u32x4 kb = z ? u32x4{0u, 0u, 0u, 0u} : score_chunk<ET>(kr[set][e]);
      const u32x4 vb = z ? u32x4{0u, 0u, 0u, 0u} : score_chunk<ET>(vr[set][e]);
      // K row-major as in the bf16 kernel's ring: piece dc at dc ^ (row % 16)
      lk[row * 16 + (dc ^ (row & (PA_PREFILL_KSWZ - 1)))] = kb;
      // V row-major as in the bf16 kernel's ring: piece dc at dc ^ 2(row % 8)
      *reinterpret_cast<u32x4*>(lv + row * (kD * 2) +
                                ((dc ^ (2 * (row & (PA_PREFILL_VSWZ - 1)))) << 4)) = vb;
    }
  };

  // A wave whose 32 rows all lie past the tile's last token (a short slice or a
  // decode row in a 128-row tile) still stages its share of every key tile but
  // computes nothing.
  const bool busy = j0 + (wave * 32) / G < j1;

  // ---- running state: lane 16g + r owns query row r of each 16-row tile -----
  f32x4 acc[2][8];
  float m[2], lsum[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    m[rt] = kNegInf;
    lsum[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int min_pos = c + j0;
  const int max_pos = kend - 1;
  const int ntiles = kend > 0 ? (kend + kKeys - 1) / kKeys : 0;
  // Sliding window: a row at position p sees p-W+1 .. p, so the walk starts at
  // the tile holding the earliest key any row of this tile sees.
  const int W = a.window;
  const int kt0 = W > 0 ? max(0, min_pos - W + 1) / kKeys : 0;
  int lo_row[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) lo_row[rt] = W > 0 ? pos[rt] - W + 1 : INT32_MIN;
  // ALiBi: slope * log2(e) of each row's query head (the scores are in log2 units)
  float slope2[2] = {0.f, 0.f};
  if constexpr (AL) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int row = wave * 32 + rt * 16 + r16;
      slope2[rt] = a.alibi[g * G + row % G] * 1.4426950408889634f;
    }
  }

  // prologue: the table window, then tile kt0 in LDS and tile kt0+1 in flight
  // (no tiles: rows before position 0, written as zeros below)
  if (ntiles > kt0) {
    load_tbl(kt0 * kKeys / BS);
    // (the query rows and the entries have landed before the walk: the walk's
    // waits then count only tile loads)
    wait_vm_lgkm<0>();
    __syncthreads();
    load_tile(0, kt0 * kKeys);
    load_tile(1, min(kt0 + 1, ntiles - 1) * kKeys);
    store_tile(0, 0);
    __syncthreads();
  }
  // one key tile; BUF (= (kt - kt0) & 1) is a constant, so every register set is static
  auto iteration = [&](int kt, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int k0 = kt * kKeys;
    // tile kt+2 into the register set tile kt used (it is in LDS already);
    // past the walk's end, its last tile again (never stored)
    const int kn = min(kt + 2, ntiles - 1);
    if ((min(kn * kKeys + kKeys, kend) - 1) / BS >= tbl0 + kTblWin) {
      // the window ends before tile kn's last block: every thread is past its
      // reads of the old one (the barrier that ended the previous step)
      load_tbl(kn * kKeys / BS);
      __syncthreads();
    }
    load_tile(buf, kn * kKeys);
    const u32x4* lk = reinterpret_cast<const u32x4*>(s_mem + buf * kBufBytes);
    const uint8_t* lv = s_mem + buf * kBufBytes + kKBytes;

    if (busy) {
    // S^T = K Q^T for both 16-key halves and both row tiles
    f32x4 s[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int h = 0; h < 2; ++h) s[rt][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int row = 16 * h + r16;
        const u32x4 kf = lk[row * 16 + ((4 * mm + grp) ^ (row & (PA_PREFILL_KSWZ - 1)))];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          s[rt][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kf), __builtin_bit_cast(bf16x8, qf[rt][mm]), s[rt][h],
              0, 0, 0);
      }
    }

    constexpr int PT = OUT_F32 ? 3 : 1;  // bf16 terms per weight
    u32x4 pf[PT][2];
    softmax_step<AL, 2, PT>(s, pf, k0, pos, lo_row, slope2, min_pos, max_pos, W, sl2, grp, m,
                            lsum, acc);

    // O^T += V^T P^T: two transposed reads give keys 4g..4g+3 and 16+4g..16+4g+3
    // of dim 16dt + (lane % 16) (the layout and reads of the bf16 kernel)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      v4s half[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 16 * hh + 4 * grp + (r16 >> 2);
        const int lc = 2 * dt + ((r16 & 3) >> 1);  // logical 16-byte piece
        const int off = row * (kD * 2) + ((lc ^ (2 * (row & (PA_PREFILL_VSWZ - 1)))) << 4) +
                        ((r16 & 1) << 3);
        half[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PA_LDS(v4s)*)((PA_LDS(uint8_t)*)lv + off));
      }
      const u32x4 vf = {
          __builtin_bit_cast(uint32_t, __builtin_shufflevector(half[0], half[0], 0, 1)),
          __builtin_bit_cast(uint32_t, __builtin_shufflevector(half[0], half[0], 2, 3)),
          __builtin_bit_cast(uint32_t, __builtin_shufflevector(half[1], half[1], 0, 1)),
          __builtin_bit_cast(uint32_t, __builtin_shufflevector(half[1], half[1], 2, 3))};
#pragma unroll
      for (int t = 0; t < PT; ++t)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, vf), __builtin_bit_cast(bf16x8, pf[t][rt]), acc[rt][dt],
              0, 0, 0);
    }
    }  // busy

    if (kt + 1 < ntiles) store_tile(buf ^ 1, buf ^ 1);
    __syncthreads();
  };
  for (int kt = kt0; kt < ntiles; kt += 2) {
    iteration(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < ntiles) iteration(kt + 1, std::integral_constant<int, 1>{});
  }

  // ---- finalise: lane 16g + r holds dims 16dt + 4g + v of row r -------------
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const float l = xor_sum<16>(lsum[rt]);
    const float inv = l > 0.f ? vsc / l : 0.f;
    if (!valid[rt]) continue;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d0 = 16 * dt + 4 * grp;
      const f32x4 o = acc[rt][dt] * inv;
      if constexpr (OUT_F32) {
        float* dst = static_cast<float*>(a.out) + row_index[rt] * kD + d0;
        *reinterpret_cast<f32x4*>(dst) = o;
      } else {
        uint16_t* dst = static_cast<uint16_t*>(a.out) + row_index[rt] * kD + d0;
        const bf16x2 lo = __builtin_convertvector((f32x2{o[0], o[1]}), bf16x2);
        const bf16x2 hi = __builtin_convertvector((f32x2{o[2], o[3]}), bf16x2);
        const u32x2 w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        *reinterpret_cast<u32x2*>(dst) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 caches: K/V tiles go from the pool straight into LDS
// ---------------------------------------------------------------------------
//
// gfx950's LDS DMA (global_load_lds_dwordx4: lane l's 16 bytes land at the
// instruction's LDS base + 16 l) fills a ring of kStages 32-key stages, each
// a K tile and a V tile of 32 rows x 256 bytes, row-major as in the pool.
// No registers hold tiles in flight and no VALU repacks them.  A lane picks
// which 16-byte piece of its row it fetches, so the pieces are stored with an
// XOR swizzle.  The LDS serves 256 bytes (64 banks) per cycle: a 16-byte read
// goes in phases of 16 lanes, which read one piece of 16 consecutive K rows,
// so K rows sit at piece c ^ (row % 16); an 8-byte transposed read goes in
// phases of 32 lanes, which read two adjacent pieces of each of 8 consecutive
// V rows, so V rows sit at piece c ^ 2(row % 8).  Each phase then touches all
// 64 banks once.
// The V^T operand of O^T = V^T P^T comes from ds_read_b64_tr_b16: within a
// 16-lane group, lane s addresses 4 dims of key row 4g + s/4 and lane i gets
// dim i of the 4 rows the group addressed - 4 keys of one dimension, in the
// k order the P^T operand already has.  V rows past the context (or of a block
// id outside the pool) are zeroed in LDS before the tile is used, so that a
// zero weight never meets a NaN.

constexpr int kStages = 3;
constexpr int kStageBytes = 2 * kKeys * kD * 2;  // K and V tiles, 16 KiB
constexpr size_t kDmaLdsBytes = size_t(kStages) * kStageBytes + kTblWin * sizeof(int32_t);

template <int ET, int BS, int G, bool OUT_F32, bool AL, int NRT>
__device__ __forceinline__ void prefill_dma_body(PrefillArgs a) {
  constexpr int TT = kRows / G;  // tokens per tile
  constexpr int NW = 8 / NRT;    // waves; each owns 16 NRT query rows
  static_assert(NRT == 2 || NRT == 4, "16-row tiles per wave");
  static_assert(ET == kBF16 || (ET == kFP8 && NW == 4), "8-bit tiles: one DMA per wave");
  // this wave's DMA instructions per tile: NRT per tensor of bf16 rows, one per
  // tensor of 8-bit rows (eight 128-byte rows)
  constexpr int kDmaPerWave = ET == kFP8 ? 2 : 2 * NRT;
  extern __shared__ __attribute__((aligned(1024))) uint8_t s_mem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwg = gridDim.x * gridDim.y;
  const int id = blockIdx.y * gridDim.x + blockIdx.x;
  const int xcd = id % 8, slot = id / 8;
  const int logical = xcd * (nwg / 8) + min(xcd, nwg % 8) + slot;
  const int t = logical % gridDim.x;
  const int g = logical / gridDim.x;
  const float sl2 = a.k_scales ? a.scale_log2 * a.k_scales[g] : a.scale_log2;
  const float vsc = a.v_scales ? a.v_scales[g] : a.v_scale;
  if (t >= a.tiles[0]) return;
  const int seq = a.tiles[1 + 2 * t];
  const int tile = a.tiles[2 + 2 * t];
  if (seq < 0 || seq >= a.num_seqs) return;

  const int32_t qs0 = min(max(a.query_start[seq], 0), a.num_tokens);
  const int32_t qs1 = min(max(a.query_start[seq + 1], 0), a.num_tokens);
  const int32_t n = qs1 - qs0;
  const int32_t max_len = a.max_blocks * BS;
  const int32_t L = min(max(a.context_lens[seq], 0), max_len);
  const int32_t c = L - n;
  const int32_t j0 = tile * TT;
  const int32_t j1 = min(j0 + TT, n);
  if (j1 <= j0) return;
  const int32_t kend = c + j1;
  const int32_t* table = a.block_tables + int64_t(seq) * a.max_blocks;

  const int r16 = lane & 15, grp = lane >> 4;
  int pos[NRT];
  bool valid[NRT];
  int64_t row_index[NRT];
  u32x4 qf[NRT][4];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int row = wave * 16 * NRT + rt * 16 + r16;
    const int tok = j0 + row / G;
    valid[rt] = tok < j1;
    const int tq = min(tok, j1 - 1);
    pos[rt] = c + tok;
    const int head = g * G + row % G;
    row_index[rt] = int64_t(qs0 + tq) * a.num_heads + head;
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + row_index[rt] * kD * 2);
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) qf[rt][mm] = qp[4 * mm + grp];
  }

  // a wave with no row before the tile's last token stages its share of every
  // key tile and computes nothing
  const bool busy = j0 + (wave * 16 * NRT) / G < j1;

  f32x4 acc[NRT][8];
  float m[NRT], lsum[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m[rt] = kNegInf;
    lsum[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int min_pos = c + j0;
  const int max_pos = kend - 1;
  const int ntiles = kend > 0 ? (kend + kKeys - 1) / kKeys : 0;
  const int W = a.window;
  const int kt0 = W > 0 ? max(0, min_pos - W + 1) / kKeys : 0;
  int lo_row[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) lo_row[rt] = W > 0 ? pos[rt] - W + 1 : INT32_MIN;
  float slope2[NRT] = {};
  if constexpr (AL) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int row = wave * 16 * NRT + rt * 16 + r16;
      slope2[rt] = a.alibi[g * G + row % G] * 1.4426950408889634f;
    }
  }

  // ---- block-table entries in LDS -------------------------------------------
  // Vector memory operations complete in order, so a table entry loaded from
  // global memory inside the walk would wait for every tile DMA issued before
  // it.  The walk reads its entries from a window of kTblWin of them in LDS
  // instead (entries outside the pool stored as -1), loaded by the whole
  // workgroup before the walk and again when the walk passes the window's end.
  int32_t* s_tbl = reinterpret_cast<int32_t*>(s_mem + kStages * kStageBytes);
  const int nblk = kend > 0 ? (kend + BS - 1) / BS : 0;
  int tbl0 = 0;  // first block the window holds
  auto load_tbl = [&](int first) {
    tbl0 = first;
    const int cnt = min(kTblWin, nblk - first);
    for (int i = tid; i < cnt; i += 64 * NW) {
      const int p = table[first + i];
      s_tbl[i] = (p < 0 || int64_t(p) >= a.num_blocks) ? -1 : p;
    }
  };
  // entry of block b, tbl0 <= b < min(tbl0 + kTblWin, nblk)
  auto entry = [&](int b) { return s_tbl[b - tbl0]; };
  load_tbl(kt0 * kKeys / BS);
  // (the query rows and the entries have landed before the walk: the walk's
  // waits then count only tile DMAs)
  wait_vm_lgkm<0>();
  __syncthreads();

  // ---- the DMA side ---------------------------------------------------------
  constexpr int kRowBytes = kD * 2;
  const int64_t blk_stride = int64_t(a.num_kv_heads) * BS * kRowBytes;
  const int64_t head_off = int64_t(g) * BS * kRowBytes;
  const int rr = lane >> 4, piece = lane & 15;  // row within a 4-row group, LDS piece
  // Wave w moves rows 4NRT w .. 4NRT (w+1) - 1 of both tiles: NRT 4-row groups,
  // each one DMA instruction (1 KiB) per tensor - 2 NRT instructions per wave
  // per tile.
  auto issue = [&](int kt, int stage) {
    const int k0 = kt * kKeys;
    if constexpr (ET == kFP8) {
      // Rows 8w .. 8w+7 of the tile, 128 bytes each (eight share a block: block
      // sizes are multiples of 8), land as they are in the upper half of the
      // stage's K and V areas; convert() expands them into the bf16 layout.
      const int r0 = 8 * wave;
      const uint32_t key0 = uint32_t(k0 + r0);
      int phys = __builtin_amdgcn_readfirstlane(entry(min(int(key0 / BS), nblk - 1)));
      phys = phys < 0 ? 0 : phys;
      const int64_t base = int64_t(phys) * (blk_stride / 2) + head_off / 2 +
                           int64_t(key0 % BS) * (kRowBytes / 2) + lane * 16;
      uint8_t* lk = s_mem + stage * kStageBytes + kKeys * kRowBytes / 2 + r0 * (kRowBytes / 2);
      uint8_t* lv = lk + kKeys * kRowBytes;
      __builtin_amdgcn_global_load_lds(a.k_pool + base, (PA_LDS(void)*)lk, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(a.v_pool + base, (PA_LDS(void)*)lv, 16, 0, 0);
      return;
    }
#pragma unroll
    for (int i = 0; i < NRT; ++i) {
      const int r0 = 4 * NRT * wave + 4 * i;  // first row of the group (wave-uniform)
      // The group's 4 keys share a block (block sizes are multiples of 4).
      // Keys past the context read rows of the sequence's last block (in
      // bounds; their scores are masked and their V rows zeroed before use).
      const uint32_t key0 = uint32_t(k0 + r0);
      int phys = __builtin_amdgcn_readfirstlane(entry(min(int(key0 / BS), nblk - 1)));
      phys = phys < 0 ? 0 : phys;
      // the group's base (scalar), then the lane's row and swizzled piece
      const int64_t base =
          int64_t(phys) * blk_stride + head_off + int64_t(key0 % BS) * kRowBytes;
      const int row = r0 + rr;
      const uint32_t ko = uint32_t(rr * kRowBytes + ((piece ^ (row & (PA_PREFILL_KSWZ - 1))) << 4));
      const uint32_t vo =
          uint32_t(rr * kRowBytes + ((piece ^ (2 * (row & (PA_PREFILL_VSWZ - 1)))) << 4));
      uint8_t* lk = s_mem + stage * kStageBytes + r0 * kRowBytes;
      uint8_t* lv = lk + kKeys * kRowBytes;
      __builtin_amdgcn_global_load_lds(a.k_pool + base + ko, (PA_LDS(void)*)lk, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(a.v_pool + base + vo, (PA_LDS(void)*)lv, 16, 0, 0);
    }
  };
  // V rows that must read as zero: past the context, or in a block outside the
  // pool (whose K rows read as zero too)
  auto fix_needed = [&](int kt) -> bool {
    const int k0 = kt * kKeys;
    if (k0 + kKeys > kend) return true;
    bool bad = false;
#pragma unroll
    for (int b = 0; b < kKeys / BS; ++b) bad |= __builtin_amdgcn_readfirstlane(entry(k0 / BS + b)) < 0;
    return bad;
  };
  auto fix = [&](int kt, int stage) {
    const int k0 = kt * kKeys;
    constexpr int PPT = 512 / (64 * NW);        // 16-byte pieces per thread (32 rows x 16)
    const int row = tid / (16 / PPT);
    const int key = k0 + row;
    const bool past = key >= kend;
    const bool out = !past && entry(key / BS) < 0;  // a block outside the pool
    u32x4* dst = reinterpret_cast<u32x4*>(s_mem + stage * kStageBytes + row * kRowBytes) +
                 PPT * (tid % (16 / PPT));
    if (past || out) {
#pragma unroll
      for (int e = 0; e < PPT; ++e) dst[kKeys * kRowBytes / 16 + e] = u32x4{0u, 0u, 0u, 0u};
    }
    if (out) {  // its keys too read as zero (the DMA brought block 0's rows)
#pragma unroll
      for (int e = 0; e < PPT; ++e) dst[e] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // 8-bit tiles: every thread expands two 8-byte halves of chunks (8 codes:
  // piece p of row r, 16 r + p = 256 i + tid) of K and of V into 16-byte bf16
  // pieces at their swizzled places, so the 16 lanes of a store cover the 16
  // pieces of one row (no bank conflict).  The codes sit where rows 16..31
  // go, so every half is read before any piece is written.  The scales are
  // applied to the scores and the outputs (codes convert to bf16 exactly).
  auto convert = [&](int stage) {
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* lk = s_mem + stage * kStageBytes;
    uint8_t* lv = lk + kKeys * kRowBytes;
    u32x2 kh[2], vh[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      kh[i] = *reinterpret_cast<const u32x2*>(lk + kKeys * kRowBytes / 2 + (256 * i + tid) * 8);
      vh[i] = *reinterpret_cast<const u32x2*>(lv + kKeys * kRowBytes / 2 + (256 * i + tid) * 8);
    }
    wait_vm_lgkm<63>();  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * i + (tid >> 4), pc = tid & 15;
      *reinterpret_cast<u32x4*>(lk + r * kRowBytes + ((pc ^ (r & (PA_PREFILL_KSWZ - 1))) << 4)) =
          score_chunk<kFP8>(kh[i]);
      *reinterpret_cast<u32x4*>(lv + r * kRowBytes +
                                ((pc ^ (2 * (r & (PA_PREFILL_VSWZ - 1)))) << 4)) =
          score_chunk<kFP8>(vh[i]);
    }
    wait_vm_lgkm<63>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: kStages-1 tiles in flight
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (kt0 + p < ntiles) issue(kt0 + p, p);

  // One key tile in ring stage STAGE (= (kt - kt0) % kStages, a constant, so
  // every LDS address is a fixed register plus an immediate offset).
  auto step = [&](int kt, auto stage_c) {
    constexpr int stage = decltype(stage_c)::value;
    // this wave's DMAs of tile kt have landed once at most 2 NRT per later tile remain
    const int later = min(kStages - 2, ntiles - 1 - kt);
    if (later >= 1)
      wait_vm_lgkm<kDmaPerWave>();
    else
      wait_vm_lgkm<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (ET == kFP8) convert(stage);
    if (fix_needed(kt)) {
      fix(kt, stage);
      wait_vm_lgkm<63>();  // lgkmcnt(0): the zeros are written before the barrier
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    // the stage tile kt-1 used is free: refill it with tile kt+kStages-1
    if (kt + kStages - 1 < ntiles) {
      const int tn = kt + kStages - 1;
      // its last block past the window: move the window to tile kt+1's first
      // block (tile kt no longer needs entries; every wave is past fix(kt))
      if ((min(tn * kKeys + kKeys, kend) - 1) / BS >= tbl0 + kTblWin) {
        __syncthreads();
        load_tbl((kt + 1) * kKeys / BS);
        __syncthreads();
      }
      constexpr int free_stage = stage == 0 ? kStages - 1 : stage - 1;
      issue(tn, free_stage);
    }
    const int k0 = kt * kKeys;
    const uint8_t* lk = s_mem + stage * kStageBytes;
    const uint8_t* lv = lk + kKeys * kRowBytes;

    if (busy) {
    // S^T = K Q^T: A = key rows (16h + r16), pieces (4mm + grp) ^ (row % 16)
    f32x4 sc4[NRT][2];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int h = 0; h < 2; ++h) sc4[rt][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 16 * h + r16;
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(
            lk + row * kRowBytes + (((4 * mm + grp) ^ (row & (PA_PREFILL_KSWZ - 1))) << 4));
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
          sc4[rt][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kf), __builtin_bit_cast(bf16x8, qf[rt][mm]),
              sc4[rt][h], 0, 0, 0);
      }
    }

    constexpr int PT = OUT_F32 ? 3 : 1;  // bf16 terms per weight
    u32x4 pf[PT][NRT];
    softmax_step<AL, NRT, PT>(sc4, pf, k0, pos, lo_row, slope2, min_pos, max_pos, W, sl2,
                              grp, m, lsum, acc);

    // O^T += V^T P^T: two transposed reads give keys 4g..4g+3 and 16+4g..16+4g+3
    // of dim 16dt + (lane % 16)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      v4s half[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 16 * hh + 4 * grp + (r16 >> 2);
        const int lc = 2 * dt + ((r16 & 3) >> 1);            // logical 16-byte piece
        const int off =
            row * kRowBytes + ((lc ^ (2 * (row & (PA_PREFILL_VSWZ - 1)))) << 4) + ((r16 & 1) << 3);
        half[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PA_LDS(v4s)*)((PA_LDS(uint8_t)*)lv + off));
      }
      const u32x4 vf = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(half[0], half[0], 0, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(half[0], half[0], 2, 3)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(half[1], half[1], 0, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(half[1], half[1], 2, 3))};
#pragma unroll
      for (int t = 0; t < PT; ++t)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
          acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, vf), __builtin_bit_cast(bf16x8, pf[t][rt]), acc[rt][dt],
              0, 0, 0);
    }
    }  // busy
  };
  static_assert(kStages == 3, "the walk is unrolled by the ring's three stages");
  for (int kt = kt0; kt < ntiles; kt += kStages) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < ntiles) step(kt + 1, std::integral_constant<int, 1>{});
    if (kt + 2 < ntiles) step(kt + 2, std::integral_constant<int, 2>{});
  }

#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const float l = xor_sum<16>(lsum[rt]);
    const float inv = l > 0.f ? vsc / l : 0.f;
    if (!valid[rt]) continue;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d0 = 16 * dt + 4 * grp;
      const f32x4 o = acc[rt][dt] * inv;
      if constexpr (OUT_F32) {
        float* dst = static_cast<float*>(a.out) + row_index[rt] * kD + d0;
        *reinterpret_cast<f32x4*>(dst) = o;
      } else {
        uint16_t* dst = static_cast<uint16_t*>(a.out) + row_index[rt] * kD + d0;
        const bf16x2 lo = __builtin_convertvector((f32x2{o[0], o[1]}), bf16x2);
        const bf16x2 hi = __builtin_convertvector((f32x2{o[2], o[3]}), bf16x2);
        const u32x2 w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        *reinterpret_cast<u32x2*>(dst) = w;
      }
    }
  }
}

template <int BS, int G, bool OUT_F32, bool AL, int NRT>
__global__ void __launch_bounds__(64 * (8 / NRT), NRT == 2 ? 2 : 1)
    prefill_dma_kernel(PrefillArgs a) {
  prefill_dma_body<kBF16, BS, G, OUT_F32, AL, NRT>(a);
}

// 8-bit caches: the same kernel, staging the codes and expanding them in LDS
template <int BS, int G, bool OUT_F32, bool AL, int NRT>
__global__ void __launch_bounds__(64 * (8 / NRT), NRT == 2 ? 2 : 1)
    prefill_dma8_kernel(PrefillArgs a) {
  prefill_dma_body<kFP8, BS, G, OUT_F32, AL, NRT>(a);
}

template <int ET, int BS, int G>
int launch_g(const PrefillArgs& a, bool out_f32, dim3 grid, hipStream_t stream) {
  const bool al = a.alibi != nullptr;
  if constexpr (ET == kBF16 && PA_PREFILL_DMA) {
    constexpr int NRT = PA_PREFILL_ROW_TILES;
    const size_t lds = kDmaLdsBytes;
    const dim3 block(64 * (8 / NRT));
    if (out_f32 && al)
      hipLaunchKernelGGL((prefill_dma_kernel<BS, G, true, true, NRT>), grid, block, lds, stream, a);
    else if (out_f32)
      hipLaunchKernelGGL((prefill_dma_kernel<BS, G, true, false, NRT>), grid, block, lds, stream, a);
    else if (al)
      hipLaunchKernelGGL((prefill_dma_kernel<BS, G, false, true, NRT>), grid, block, lds, stream, a);
    else
      hipLaunchKernelGGL((prefill_dma_kernel<BS, G, false, false, NRT>), grid, block, lds, stream, a);
    return launch_result("pa_prefill");
  } else if constexpr (ET == kFP8 && PA_PREFILL_DMA_FP8) {
    const size_t lds = kDmaLdsBytes;
    const dim3 block(256);
    if (out_f32 && al)
      hipLaunchKernelGGL((prefill_dma8_kernel<BS, G, true, true, 2>), grid, block, lds, stream, a);
    else if (out_f32)
      hipLaunchKernelGGL((prefill_dma8_kernel<BS, G, true, false, 2>), grid, block, lds, stream, a);
    else if (al)
      hipLaunchKernelGGL((prefill_dma8_kernel<BS, G, false, true, 2>), grid, block, lds, stream, a);
    else
      hipLaunchKernelGGL((prefill_dma8_kernel<BS, G, false, false, 2>), grid, block, lds, stream, a);
    return launch_result("pa_prefill");
  } else {
    const size_t lds = 2 * kBufBytes + kTblWin * sizeof(int32_t);
    if (out_f32 && al)
      hipLaunchKernelGGL((prefill_kernel<ET, BS, G, true, true>), grid, dim3(256), lds, stream, a);
    else if (out_f32)
      hipLaunchKernelGGL((prefill_kernel<ET, BS, G, true, false>), grid, dim3(256), lds, stream, a);
    else if (al)
      hipLaunchKernelGGL((prefill_kernel<ET, BS, G, false, true>), grid, dim3(256), lds, stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<ET, BS, G, false, false>), grid, dim3(256), lds, stream,
                         a);
    return launch_result("pa_prefill");
  }
}

template <int ET, int BS>
int launch_bs(const PrefillArgs& a, int group, bool out_f32, dim3 grid, hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<ET, BS, 1>(a, out_f32, grid, stream);
    case 2: return launch_g<ET, BS, 2>(a, out_f32, grid, stream);
    case 3: return launch_g<ET, BS, 3>(a, out_f32, grid, stream);
    case 4: return launch_g<ET, BS, 4>(a, out_f32, grid, stream);
    case 5: return launch_g<ET, BS, 5>(a, out_f32, grid, stream);
    case 6: return launch_g<ET, BS, 6>(a, out_f32, grid, stream);
    case 7: return launch_g<ET, BS, 7>(a, out_f32, grid, stream);
    case 8: return launch_g<ET, BS, 8>(a, out_f32, grid, stream);
    default: return launch_g<ET, BS, 16>(a, out_f32, grid, stream);
  }
}

template <int ET>
int launch_et(const PrefillArgs& a, int block_size, int group, bool out_f32, dim3 grid,
              hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_bs<ET, 8>(a, group, out_f32, grid, stream);
    case 16: return launch_bs<ET, 16>(a, group, out_f32, grid, stream);
    default: return launch_bs<ET, 32>(a, group, out_f32, grid, stream);
  }
}

// Query heads per KV head the prefill kernels take.
constexpr bool prefill_group_supported(int g) { return (g >= 1 && g <= 8) || g == 16; }

// Launch the attention kernel of one cache type (the instantiations live in
// pa_prefill_bf16.hip and pa_prefill_fp8.hip, compiled apart).
int launch_prefill_bf16(const PrefillArgs& a, int block_size, int group, bool out_f32,
                        dim3 grid, hipStream_t stream);
int launch_prefill_fp8(const PrefillArgs& a, int block_size, int group, bool out_f32,
                       dim3 grid, hipStream_t stream);


}  // namespace pf
}  // namespace pa
