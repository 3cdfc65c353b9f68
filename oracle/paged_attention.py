"""Plain float64 CPU oracle of paged attention decode and its KV writes.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module. It shares no code with the HIP library and imports nothing
from it.

The method (paged attention, as described on the five pages this work follows)
changes only *where* a sequence's keys and values live: the KV cache is cut into
fixed-size physical blocks, and a per-sequence block table maps logical block j
to a physical block. Attention itself is the textbook one. So this oracle is
that definition written out plainly:

1. gather the sequence's key/value rows in logical order through the block
   table (the indexing rule of "How Paged Attention and Continuous Batching
   Actually Work", section "Paged attention: virtual memory for the KV cache";
   "LLM paged attention arch", section "The architecture: every piece
   explained", which states that table entry i backs logical tokens
   [16i, 16i+15]);
2. score every past token with q.k / sqrt(d_k) ("Paged Attention as a Memory
   Manager", section "How the Kernel Executes Paged Attention");
3. subtract the maximum score, exponentiate, normalise, and take the weighted
   sum of value rows (same section, "Softmax and output reduction"; "PagedAttention
   and continuous batching", section "Attention kernel modification").

The oracle deliberately uses the two-pass form (max first, then the weighted
sum); the GPU kernels use a running softmax, which is the same function in exact
arithmetic.

Storage conventions (shared with the caller only as array shapes):

* A KV pool is an array ``[num_blocks][num_kv_heads][block_size][head_dim]``.
  K and V live in two separate pools of that shape.
* Values of dtype ``"f32"`` are ``numpy.float32`` arrays; values of dtype
  ``"bf16"`` are ``numpy.uint16`` arrays holding bfloat16 bit patterns.
* An 8-bit cache (dtype ``"fp8"``) holds ``numpy.uint8`` E4M3 codes; stored
  code c stands for e4m3(c) * scale, with one scale for the K pool and one for
  the V pool.  Its queries and new tokens are bfloat16 bit patterns.
* ``block_tables`` is ``[num_seqs][max_blocks]`` of int32; only the first
  ceil(L_i / block_size) entries of row i are ever read.
* ``context_lens[i]`` = L_i counts every token sequence i attends to, including
  the token appended this step.
* Query head h belongs to KV head h // G, with G = num_heads / num_kv_heads
  (contiguous query-head groups; the pages only name grouped-query attention).
"""

from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# Value decoding (exact)
# ---------------------------------------------------------------------------

def to_f64(values, dtype: str) -> np.ndarray:
    """Widen stored values to float64 without rounding.

    bfloat16 is the upper half of an IEEE binary32, so its bit pattern shifted
    left by 16 is the binary32 with the same value; binary32 widens exactly to
    binary64.
    """
    if dtype == "f32":
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(values, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN
            return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# 8-bit E4M3 values (the fp8 KV cache)
# ---------------------------------------------------------------------------
#
# The pages name an 8-bit KV cache only as a lever on top of paging: it halves
# the bytes of every block ("PagedAttention" glossary page, section "What
# paging costs") and relieves a full block pool ("How Paged Attention and
# Continuous Batching Actually Work", section "What this means when you serve
# a model").  They fix no format or scaling.  The format taken here is OCP
# E4M3 ("FN": no infinities): 1 sign bit, 4 exponent
# bits with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
# m/8 * 2^-6; the all-ones pattern S.1111.111 is NaN; the largest finite
# magnitude is 1.75 * 2^8 = 448.

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Exact value of one E4M3 byte (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return math.nan
    if exponent == 0:
        return sign * math.ldexp(mantissa, -9)  # (m/8) * 2^-6
    return sign * math.ldexp(8 + mantissa, exponent - 10)  # (1 + m/8) * 2^(e-7)


_E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def fp8_to_f64(codes) -> np.ndarray:
    """Widen E4M3 codes to float64 (exact: every E4M3 value is a float64)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# The 127 non-negative finite values, in code order 0x00..0x7E (increasing).
_E4M3_MAGNITUDES = _E4M3_TABLE[:0x7F]


def fp8_encode(values) -> np.ndarray:
    """E4M3 codes of the given values: round to nearest, ties to the even code.

    Magnitudes above 448 saturate to 448 (the format has no infinity; this
    library clamps instead of producing NaN), NaN becomes S.1111.111, and the
    sign bit follows the sign of the value (so -0.0 and negative values that
    round to zero give 0x80).  Nearest is found by direct search over the 127
    finite magnitudes; of two equally near neighbours the one whose code is
    even (mantissa bit 0 clear) wins.
    """
    y = np.asarray(values, dtype=np.float64)
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for n, v in enumerate(flat):
        sign = 0x80 if math.copysign(1.0, v) < 0 else 0
        if math.isnan(v):
            out[n] = sign | 0x7F
            continue
        a = abs(v)
        if a >= E4M3_MAX:
            out[n] = sign | 0x7E
            continue
        hi = int(np.searchsorted(_E4M3_MAGNITUDES, a, side="left"))  # first magnitude >= a
        if _E4M3_MAGNITUDES[hi] == a:
            code = hi
        else:
            lo = hi - 1
            below, above = a - _E4M3_MAGNITUDES[lo], _E4M3_MAGNITUDES[hi] - a
            if below < above:
                code = lo
            elif above < below:
                code = hi
            else:
                code = lo if lo % 2 == 0 else hi
        out[n] = sign | code
    return out.reshape(y.shape)


def fp8_quantize(bf16_bits, scale: float) -> np.ndarray:
    """E4M3 codes stored for bfloat16 inputs with dequantisation scale ``scale``.

    Each input x is widened exactly to binary32, divided by the scale in
    binary32 (IEEE division, rounded to nearest), and the quotient is encoded
    with :func:`fp8_encode`.
    """
    x32 = to_f64(bf16_bits, "bf16").astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):  # IEEE: overflow gives +-inf
        y32 = x32 / np.float32(scale)
    return fp8_encode(y32.astype(np.float64))


def _kv_f64(rows, dtype: str, scale: float) -> np.ndarray:
    """Exact float64 values of stored K or V rows (E4M3 codes times the pool's scale)."""
    if dtype == "fp8":
        return fp8_to_f64(rows) * float(scale)
    return to_f64(rows, dtype)


def head_scale(scale, kv_head: int) -> float:
    """The scale of KV head ``kv_head``: one number for the whole pool, or one
    per KV head (a sequence indexed by head)."""
    return float(scale) if np.ndim(scale) == 0 else float(scale[kv_head])


def _q_dtype(dtype: str) -> str:
    return "bf16" if dtype == "fp8" else dtype


# ---------------------------------------------------------------------------
# Block arithmetic
# ---------------------------------------------------------------------------

def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks held by a sequence of ``num_tokens`` tokens: ceil(t / B).

    "How Paged Attention and Continuous Batching Actually Work", section "Paged
    attention: virtual memory for the KV cache" (a request with t tokens holds
    ceil(t/16) blocks).
    """
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("num_tokens must be >= 0 and block_size > 0")
    return -(-num_tokens // block_size)


def last_block_waste(num_tokens: int, block_size: int) -> int:
    """Unused token slots in the sequence's last block: B*ceil(t/B) - t.

    Same section: the waste is bounded by one partial block, i.e. at most B-1
    slots (15 for 16-token blocks).
    """
    return blocks_needed(num_tokens, block_size) * block_size - num_tokens


def slot_of(table_row, position: int, block_size: int) -> int:
    """Flat slot of logical token ``position`` of one sequence.

    The indexing rule of "How Paged Attention and Continuous Batching Actually
    Work", section "Paged attention: virtual memory for the KV cache" (the
    formula itself is lost from the extracted page; its prose survives): divide
    the position by the block size to find the logical block, look up the
    physical block in the table, multiply by the block size and add the offset
    inside the block.  The slot s addresses row (s // B, s % B) of the pool.
    """
    logical_block = position // block_size
    offset = position % block_size
    return int(table_row[logical_block]) * block_size + offset


def gather_rows(pool: np.ndarray, table_row, length: int, block_size: int,
                kv_head: int) -> np.ndarray:
    """Rows 0..length-1 of one KV head of one sequence, in logical order.

    Returns the stored values (no conversion), shape ``[length][head_dim]``.
    Follows the block-level loop of "Paged Attention as a Memory Manager",
    section "How the Kernel Executes Paged Attention": for every logical block,
    read its physical block from the table, then read the rows inside it.
    Only rows of positions < length are read, which is the padding mask of the
    same section applied before anything is computed.
    """
    if pool.shape[2] != block_size:
        raise ValueError("pool block dimension does not match block_size")
    pieces = [pool[:0, kv_head, 0, :]]
    for logical_block in range(blocks_needed(length, block_size)):
        physical_block = int(table_row[logical_block])
        rows_here = min(block_size, length - logical_block * block_size)
        pieces.append(pool[physical_block, kv_head, :rows_here, :])
    return np.concatenate(pieces)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _check_shapes(q, k_pool, v_pool, block_tables, context_lens):
    num_seqs, num_heads, head_dim = q.shape
    num_blocks, num_kv_heads, block_size, head_dim_k = k_pool.shape
    if v_pool.shape != k_pool.shape:
        raise ValueError("K and V pools differ in shape")
    if head_dim_k != head_dim:
        raise ValueError("head_dim of q and of the pools differ")
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    if len(block_tables) != num_seqs or len(context_lens) != num_seqs:
        raise ValueError("one block-table row and one context length per sequence")
    return num_seqs, num_heads, head_dim, num_kv_heads, block_size


def _softmax_weighted_sum(scores: np.ndarray, values: np.ndarray):
    """Two-pass softmax-weighted sum of value rows.

    "Paged Attention as a Memory Manager", section "How the Kernel Executes
    Paged Attention" (softmax and output reduction): reduce to the maximum
    score for numerical stability, then accumulate the weighted sum of value
    vectors.  Returns (output, max_score, sum_of_weights).
    """
    m = scores.max()
    w = np.exp(scores - m)
    total = w.sum()
    return (w @ values) / total, m, total


def decode(q, k_pool, v_pool, block_tables, context_lens, scale: float,
           dtype: str, k_scale: float = 1.0, v_scale: float = 1.0, window: int = 0,
           alibi_slopes=None) -> np.ndarray:
    """Decode attention of one query token per sequence over a paged KV cache.

    For sequence i and query head h (KV head g = h // G):
        s_t = scale * q[i,h] . k_t        for t < L_i
        out[i,h] = sum_t softmax(s)_t * v_t
    with k_t, v_t gathered through ``block_tables[i]``.  Score and scale are
    those of "Paged Attention as a Memory Manager", section "How the Kernel
    Executes Paged Attention"; the attended range K_{0:t} is that of
    "PagedAttention and continuous batching", section "Attention kernel
    modification".  A sequence with L_i = 0 gets an all-zero output (the pages
    never produce one; decode always has the new token).  For an 8-bit cache
    (``dtype="fp8"``) k_t and v_t are the stored codes' values times
    ``k_scale`` / ``v_scale`` and q holds bfloat16 bit patterns.  ``window``
    and ``alibi_slopes`` select the attention variants of :func:`attended_range`
    and :func:`alibi_bias` (defaults: neither).

    Returns float64 ``[num_seqs][num_heads][head_dim]``.
    """
    num_seqs, num_heads, head_dim, num_kv_heads, block_size = _check_shapes(
        q, k_pool, v_pool, block_tables, context_lens)
    group = num_heads // num_kv_heads
    q64 = to_f64(q, _q_dtype(dtype))
    out = np.zeros((num_seqs, num_heads, head_dim), dtype=np.float64)
    for i in range(num_seqs):
        length = int(context_lens[i])
        if length == 0:
            continue
        for g in range(num_kv_heads):
            keys = _kv_f64(gather_rows(k_pool, block_tables[i], length, block_size, g),
                           dtype, head_scale(k_scale, g))
            values = _kv_f64(gather_rows(v_pool, block_tables[i], length, block_size, g),
                             dtype, head_scale(v_scale, g))
            lo, hi = attended_range(length - 1, window)
            for h in range(g * group, (g + 1) * group):
                scores = scale * (keys[lo:hi] @ q64[i, h])
                scores = scores + alibi_bias(alibi_slopes, h, lo, hi, length - 1)
                out[i, h], _, _ = _softmax_weighted_sum(scores, values[lo:hi])
    return out


def attended_range(position: int, window: int = 0):
    """Positions [lo, hi) a query at ``position`` attends to.

    Causal attention sees 0..position ("PagedAttention and continuous
    batching", section "Attention kernel modification").  A sliding window of W
    tokens - one of the variants "Paged Attention as a Memory Manager", section
    "When It Falls Down", names - keeps the last W of them, position-W+1 ..
    position (the window's usual definition: a token sees itself and the W-1
    before it).  window = 0 means no window.
    """
    if window < 0:
        raise ValueError("window must be >= 0")
    hi = visible_keys(position)
    lo = max(0, position - window + 1) if window else 0
    return lo, hi


def alibi_bias(slopes, head: int, lo: int, hi: int, position: int):
    """ALiBi score bias of keys lo..hi-1 for a query at ``position`` (0 if no slopes).

    ALiBi, the other variant the same passage names, adds to each score a
    penalty linear in the key's distance from the query: slope_h * (t - position)
    for key t and query head h (Press, Smith and Lewis, "Train Short, Test Long:
    Attention with Linear Biases").
    """
    if slopes is None:
        return 0.0
    t = np.arange(lo, hi, dtype=np.float64)
    return float(slopes[head]) * (t - position)


def alibi_slopes(num_heads: int) -> np.ndarray:
    """The geometric ALiBi slopes of the paper for a power-of-two head count:
    head h (from 0) gets 2^(-8 (h+1) / num_heads)."""
    if num_heads <= 0 or num_heads & (num_heads - 1):
        raise ValueError("num_heads must be a power of two")
    return np.array([2.0 ** (-8.0 * (h + 1) / num_heads) for h in range(num_heads)])


def query_position(context_len: int, num_query: int, j: int) -> int:
    """Position of the j-th of a sequence's ``num_query`` query tokens.

    A step computes a sequence's last ``num_query`` tokens: the KV of all
    earlier positions (a cached prefix, earlier prompt slices or earlier
    decode steps) is already in the cache, and this step's own tokens are
    written before attention, so the sequence holds ``context_len`` tokens and
    query token j sits at position context_len - num_query + j.
    """
    return context_len - num_query + j


def visible_keys(position: int) -> int:
    """Keys a query at ``position`` attends to under the causal rule: 0..position."""
    return position + 1


def prefill(q, k_pool, v_pool, block_tables, query_start, context_lens, scale: float,
            dtype: str, k_scale: float = 1.0, v_scale: float = 1.0, window: int = 0,
            alibi_slopes=None) -> np.ndarray:
    """Causal attention of every scheduled query token of a mixed batch.

    The batch is one flattened sequence of query tokens: sequence i owns rows
    ``query_start[i] .. query_start[i+1]-1`` of ``q`` (``[num_tokens][Hq][D]``),
    and metadata says where each request's tokens begin and end and which
    positions they may look at ("How Paged Attention and Continuous Batching
    Actually Work", section "Continuous batching: schedule steps, not
    batches").  Query token j of sequence i sits at position
    p = :func:`query_position` (L_i, n_i, j) and attends causally to positions
    0..p, whose K/V rows are gathered block by block through the table
    ("PagedAttention and continuous batching", section "Attention kernel
    modification"); scores and softmax are those of :func:`decode`.  A decode
    row is the case n_i = 1 (p = L_i - 1).  Rows with p < 0 (more query tokens
    than context: a caller error) are left zero.  ``window`` and
    ``alibi_slopes`` select the variants of :func:`attended_range` and
    :func:`alibi_bias`.

    Returns float64 ``[num_tokens][num_heads][head_dim]``.
    """
    num_heads = q.shape[1]
    num_blocks, num_kv_heads, block_size, head_dim = k_pool.shape
    if q.ndim != 3 or q.shape[2] != head_dim or num_heads % num_kv_heads:
        raise ValueError("q must be [num_tokens][num_heads][head_dim] with num_heads % num_kv_heads == 0")
    starts = [int(x) for x in query_start]
    num_seqs = len(starts) - 1
    if num_seqs != len(context_lens) or starts[0] != 0 or starts[-1] != q.shape[0] or \
            any(b < a for a, b in zip(starts, starts[1:])):
        raise ValueError("query_start must rise from 0 to num_tokens, one entry per sequence + 1")
    group = num_heads // num_kv_heads
    q64 = to_f64(q, _q_dtype(dtype))
    out = np.zeros((q.shape[0], num_heads, head_dim), dtype=np.float64)
    for i in range(num_seqs):
        length, n = int(context_lens[i]), starts[i + 1] - starts[i]
        if n == 0 or length == 0:
            continue
        for g in range(num_kv_heads):
            keys = _kv_f64(gather_rows(k_pool, block_tables[i], length, block_size, g),
                           dtype, head_scale(k_scale, g))
            values = _kv_f64(gather_rows(v_pool, block_tables[i], length, block_size, g),
                             dtype, head_scale(v_scale, g))
            for j in range(n):
                p = query_position(length, n, j)
                if p < 0:
                    continue
                lo, hi = attended_range(p, window)
                for h in range(g * group, (g + 1) * group):
                    scores = scale * (keys[lo:hi] @ q64[starts[i] + j, h])
                    scores = scores + alibi_bias(alibi_slopes, h, lo, hi, p)
                    out[starts[i] + j, h], _, _ = _softmax_weighted_sum(scores, values[lo:hi])
    return out


def decode_partitions(q, k_pool, v_pool, block_tables, context_lens, scale: float,
                      dtype: str, partition_size: int, max_parts: int | None = None,
                      k_scale: float = 1.0, v_scale: float = 1.0):
    """Per-partition attention results for split-KV decode.

    The pages never split a sequence's context; this follows the split-KV
    reading used by this library: partition p of sequence i covers positions
    [p*P, min((p+1)*P, L_i)).  For each (i, h, p) it returns

        part_out  = softmax-weighted sum of v_t over the partition,
        part_max  = max of the partition's scores s_t (natural units),
        part_sum  = sum over the partition of exp(s_t - part_max).

    An empty partition has part_out = 0, part_max = -inf, part_sum = 0.
    Returns three float64 arrays shaped [S][Hq][max_parts][D], [S][Hq][max_parts]
    and [S][Hq][max_parts].
    """
    num_seqs, num_heads, head_dim, num_kv_heads, block_size = _check_shapes(
        q, k_pool, v_pool, block_tables, context_lens)
    if partition_size <= 0:
        raise ValueError("partition_size must be positive")
    group = num_heads // num_kv_heads
    if max_parts is None:
        max_parts = max([blocks_needed(int(n), partition_size) for n in context_lens] + [1])
    q64 = to_f64(q, _q_dtype(dtype))
    part_out = np.zeros((num_seqs, num_heads, max_parts, head_dim), dtype=np.float64)
    part_max = np.full((num_seqs, num_heads, max_parts), -np.inf, dtype=np.float64)
    part_sum = np.zeros((num_seqs, num_heads, max_parts), dtype=np.float64)
    for i in range(num_seqs):
        length = int(context_lens[i])
        nparts = blocks_needed(length, partition_size)
        if nparts > max_parts:
            raise ValueError("max_parts too small for context_lens")
        for g in range(num_kv_heads):
            keys = _kv_f64(gather_rows(k_pool, block_tables[i], length, block_size, g),
                           dtype, head_scale(k_scale, g))
            values = _kv_f64(gather_rows(v_pool, block_tables[i], length, block_size, g),
                             dtype, head_scale(v_scale, g))
            for h in range(g * group, (g + 1) * group):
                scores = scale * (keys @ q64[i, h])
                for p in range(nparts):
                    lo, hi = p * partition_size, min((p + 1) * partition_size, length)
                    o, m, total = _softmax_weighted_sum(scores[lo:hi], values[lo:hi])
                    part_out[i, h, p] = o
                    part_max[i, h, p] = m
                    part_sum[i, h, p] = total
    return part_out, part_max, part_sum


def splitkv_merge(part_out, part_max, part_sum, context_lens, partition_size: int):
    """Merge per-partition results with their log-sum-exp weights.

    Not on the pages (they describe one running softmax over the whole
    context); this is the exact regrouping of that softmax over partitions:
        M   = max_p part_max[p]
        w_p = part_sum[p] * exp(part_max[p] - M)
        out = sum_p w_p * part_out[p] / sum_p w_p
        lse = M + ln(sum_p w_p)
    over the ceil(L_i / P) partitions sequence i has; partitions with
    part_sum = 0 get weight 0.  A sequence with L_i = 0 gets out = 0 and
    lse = -inf.  Returns (out [S][Hq][D], lse [S][Hq]) in float64.
    """
    part_out = np.asarray(part_out, dtype=np.float64)
    part_max = np.asarray(part_max, dtype=np.float64)
    part_sum = np.asarray(part_sum, dtype=np.float64)
    num_seqs, num_heads, max_parts, head_dim = part_out.shape
    out = np.zeros((num_seqs, num_heads, head_dim), dtype=np.float64)
    lse = np.full((num_seqs, num_heads), -np.inf, dtype=np.float64)
    for i in range(num_seqs):
        nparts = blocks_needed(int(context_lens[i]), partition_size)
        if nparts > max_parts:
            raise ValueError("context_lens need more partitions than part_out holds")
        for h in range(num_heads):
            live = [p for p in range(nparts) if part_sum[i, h, p] > 0]
            if not live:
                continue
            big_m = max(part_max[i, h, p] for p in live)
            weights = np.array([part_sum[i, h, p] * math.exp(part_max[i, h, p] - big_m) for p in live])
            total = weights.sum()
            out[i, h] = (weights @ part_out[i, h, live]) / total
            lse[i, h] = big_m + math.log(total)
    return out, lse


# ---------------------------------------------------------------------------
# KV writes (byte-exact)
# ---------------------------------------------------------------------------

def _quantize_heads(rows, scale) -> np.ndarray:
    """fp8_quantize of [n][num_kv_heads][head_dim] rows, head by head."""
    rows = np.asarray(rows)
    if np.ndim(scale) == 0:
        return fp8_quantize(rows, scale)
    out = np.empty(rows.shape, dtype=np.uint8)
    for g in range(rows.shape[1]):
        out[:, g, :] = fp8_quantize(rows[:, g, :], float(scale[g]))
    return out


def kv_append(k_pool, v_pool, k_new, v_new, slot_mapping, fp8_scales=None):
    """Pools after writing each new token's K/V rows at its slot.

    "How Paged Attention and Continuous Batching Actually Work", section "One
    step, end to end" (the forward pass writes KV through the slot mapping);
    "LLM paged attention arch", section "The architecture: every piece
    explained" (the new token's K/V go into the right physical block).  Token n
    with slot s >= 0 overwrites row (s // B, :, s % B, :) of both pools with
    ``k_new[n]`` / ``v_new[n]`` (all KV heads), bit for bit; a negative slot
    means "no write".  Every other byte stays as it was.  Two tokens with the
    same slot are a caller error.

    With ``fp8_scales = (k_scale, v_scale)`` the pools are an 8-bit cache and
    k_new / v_new hold bfloat16 bit patterns: each row is stored as
    :func:`fp8_quantize` of it with the pool's scale instead of a bit copy.  A
    scale may also be one per KV head (a sequence indexed by head), each head's
    rows then quantised with their own.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    if fp8_scales is not None:
        k_new = _quantize_heads(k_new, fp8_scales[0])
        v_new = _quantize_heads(v_new, fp8_scales[1])
    block_size = k_pool.shape[2]
    slots = [int(s) for s in slot_mapping]
    live = [s for s in slots if s >= 0]
    if len(set(live)) != len(live):
        raise ValueError("slot_mapping has a repeated slot")
    for n, s in enumerate(slots):
        if s < 0:
            continue
        k_out[s // block_size, :, s % block_size, :] = k_new[n]
        v_out[s // block_size, :, s % block_size, :] = v_new[n]
    return k_out, v_out


def copy_blocks(k_pool, v_pool, pairs):
    """Pools after the copy step of copy-on-write.

    "Paged Attention as a Memory Manager", section "Prefix Caching and
    Copy-on-Write": on a write to a shared block the runtime allocates a fresh
    physical block and copies the existing content into it (refcount and table
    updates are the block manager's, not this copy's).  Each (src, dst) pair
    copies every KV head and row of block src to block dst in both pools, bit
    for bit, from the state before any copy.  Destinations must be distinct and
    no destination may also be a source.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    pairs = [(int(a), int(b)) for a, b in pairs]
    dsts = [b for _, b in pairs]
    if len(set(dsts)) != len(dsts) or set(dsts) & {a for a, _ in pairs}:
        raise ValueError("copy pairs need distinct destinations that are not sources")
    for src, dst in pairs:
        k_out[dst] = k_pool[src]
        v_out[dst] = v_pool[src]
    return k_out, v_out
