"""Python binding of libpagedattn (ctypes; argument marshalling only).

Each function takes device tensors, passes their pointers and sizes to the C
entry point of the same name in ``libpagedattn.so`` and raises
:class:`PagedAttnError` on a non-OK status.  Nothing here computes: every step
runs in the library's HIP kernels, on the caller's current HIP stream unless a
stream is given.  Loading fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")
# A different build of the same library to load instead (the sanitized CPU
# test build, for instance); the in-tree library when unset.
LIB_OVERRIDE = os.environ.get("PAGEDATTN_LIB")

PA_OK = 0
PA_F32 = 0
PA_BF16 = 1
PA_FP8_E4M3 = 2
PA_SWAP_OUT = 0
PA_SWAP_IN = 1
STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED",
                4: "PA_ERR_WORKSPACE", 5: "PA_ERR_LAUNCH", 6: "PA_ERR_ID", 7: "PA_ERR_STATE",
                8: "PA_ERR_NOMEM"}

# Every symbol include/pagedattn.h and include/pa_block_manager.h declare.
EXPORTED = ("pa_abi_version", "pa_hip_runtime_version", "pa_last_error", "pa_kv_append",
            "pa_copy_blocks", "pa_swap_blocks", "pa_decode", "pa_decode_append",
            "pa_decode_static",
            "pa_decode_workspace_bytes", "pa_decode_workspace_size",
            "pa_decode_partitions", "pa_splitkv_reduce", "pa_partials_bytes", "pa_prefill",
            "pa_prefill_workspace_bytes", "pa_probe_stream_read",
            "pa_bm_create", "pa_bm_destroy", "pa_bm_add_request", "pa_bm_append_tokens",
            "pa_bm_append_batch",
            "pa_bm_fork", "pa_bm_finish", "pa_bm_schedule", "pa_bm_get_stats",
            "pa_bm_request_info", "pa_bm_blocks", "pa_bm_refcounts", "pa_bm_free_list")


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class PaCache(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int64), ("num_kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("k_scales", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p)]


class PaAttnVariant(ctypes.Structure):
    _fields_ = [("sliding_window", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("alibi_slopes", ctypes.c_void_p)]


class PaBmConfig(ctypes.Structure):
    _fields_ = [("num_gpu_blocks", ctypes.c_int64), ("num_cpu_blocks", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("prefix_caching", ctypes.c_int32),
                ("preempt_mode", ctypes.c_int32), ("watermark_blocks", ctypes.c_int32)]


_P64, _P32 = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)


class PaStepPlan(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("num_cow", ctypes.c_int32),
                ("num_swap_out", ctypes.c_int32), ("num_swap_in", ctypes.c_int32),
                ("num_preempted", ctypes.c_int32),
                ("seq_ids", _P64), ("query_start", _P32), ("context_lens", _P32),
                ("slot_mapping", _P64), ("block_tables", _P32), ("cow_pairs", _P64),
                ("swap_out_pairs", _P64), ("swap_in_pairs", _P64), ("preempted_ids", _P64),
                ("preempted_modes", _P32)]


_BM_STATS = ("free_gpu_blocks", "free_cpu_blocks", "cached_blocks", "running", "waiting",
             "swapped", "preemptions", "swapped_out_blocks", "swapped_in_blocks", "cow_copies",
             "prefix_hit_tokens", "admitted_tokens")


class PaBmStats(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in _BM_STATS]


class PaRequestInfo(ctypes.Structure):
    _fields_ = [("state", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("arrival", ctypes.c_int64), ("num_tokens", ctypes.c_int64),
                ("computed", ctypes.c_int64), ("num_blocks", ctypes.c_int64),
                ("num_cpu_blocks", ctypes.c_int64)]


_lib = None
_vp, _i32, _i64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SIGNATURES = {
    "pa_abi_version": (_i32, []),
    "pa_hip_runtime_version": (_i32, []),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_kv_append": (ctypes.c_int, [ctypes.POINTER(PaCache), _vp, _vp, _vp, _i32, _vp]),
    "pa_copy_blocks": (ctypes.c_int, [ctypes.POINTER(PaCache), _vp, _i32, _vp]),
    "pa_swap_blocks": (ctypes.c_int, [ctypes.POINTER(PaCache), _vp, _vp, _i64, _vp, _i32, _i32,
                                      _vp]),
    "pa_decode": (ctypes.c_int, [ctypes.POINTER(PaCache), _vp, _vp, _vp, _i32, _i32, _i32, _f32,
                                 ctypes.POINTER(PaAttnVariant), _vp, _i32, _vp, ctypes.c_size_t,
                                 _vp]),
    "pa_decode_static": (ctypes.c_int, [ctypes.POINTER(PaCache), _vp, _vp, _vp, _i32, _i32,
                                        _i32, _f32, ctypes.POINTER(PaAttnVariant), _vp, _i32,
                                        _vp]),
    "pa_decode_append": (ctypes.c_int, [ctypes.POINTER(PaCache), _vp, _vp, _vp, _vp, _vp, _i32,
                                        _i32, _i32, _f32, ctypes.POINTER(PaAttnVariant), _vp,
                                        _i32, _vp, ctypes.c_size_t, _vp]),
    "pa_decode_workspace_bytes": (ctypes.c_size_t, [_i32, _i32, _i32]),
    "pa_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(PaCache), _i32, _i32]),
    "pa_decode_partitions": (ctypes.c_int, [ctypes.POINTER(PaCache), _vp, _vp, _vp, _i32, _i32,
                                            _i32, _f32, _i32, _vp, _vp, _vp, _i32, _vp]),
    "pa_splitkv_reduce": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp,
                                         _i32, _vp, _vp]),
    "pa_partials_bytes": (ctypes.c_size_t, [_i32, _i32, _i32, _i32]),
    "pa_prefill": (ctypes.c_int, [ctypes.POINTER(PaCache), _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                  _i32, _f32, ctypes.POINTER(PaAttnVariant), _vp, _i32, _vp,
                                  ctypes.c_size_t, _vp]),
    "pa_prefill_workspace_bytes": (ctypes.c_size_t, [_i32, _i32, _i32, _i32]),
    "pa_probe_stream_read": (ctypes.c_int, [_vp, ctypes.c_size_t, _i32, _i32, _vp, _vp]),
    "pa_bm_create": (ctypes.c_int, [ctypes.POINTER(PaBmConfig), ctypes.POINTER(_vp)]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_add_request": (ctypes.c_int, [_vp, _i64, _vp, _i64]),
    "pa_bm_append_tokens": (ctypes.c_int, [_vp, _i64, _vp, _i64]),
    "pa_bm_append_batch": (ctypes.c_int, [_vp, _vp, _vp, _i64]),
    "pa_bm_fork": (ctypes.c_int, [_vp, _i64, _i64]),
    "pa_bm_finish": (ctypes.c_int, [_vp, _i64]),
    "pa_bm_schedule": (ctypes.c_int, [_vp, _i64, ctypes.POINTER(PaStepPlan)]),
    "pa_bm_get_stats": (ctypes.c_int, [_vp, ctypes.POINTER(PaBmStats)]),
    "pa_bm_request_info": (ctypes.c_int, [_vp, _i64, ctypes.POINTER(PaRequestInfo)]),
    "pa_bm_blocks": (ctypes.c_int, [_vp, _i64, _i32, _vp, _i64, ctypes.POINTER(_i64)]),
    "pa_bm_refcounts": (ctypes.c_int, [_vp, _vp, _i64]),
    "pa_bm_free_list": (ctypes.c_int, [_vp, _i32, _vp, _i64, ctypes.POINTER(_i64)]),
}


def load(path: str | None = None):
    """Load libpagedattn.so (after torch, so it binds to torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_OVERRIDE or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_93_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != PA_OK:
        raise PagedAttnError(status, load().pa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    """pa_dtype of a tensor; E4M3 codes come as float8_e4m3fn or uint8 tensors."""
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return PA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _token_dtype(cache) -> torch.dtype:
    """dtype of q and of new tokens for a cache: bf16 for an 8-bit cache."""
    return {PA_F32: torch.float32, PA_BF16: torch.bfloat16, PA_FP8_E4M3: torch.bfloat16}[cache.dtype]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _on_device(**tensors):
    """Every named tensor that is not None lives on a GPU (a host tensor's
    pointer handed to a kernel would fault the device)."""
    for name, t in tensors.items():
        _require(t is None or t.device.type == "cuda", f"{name} must be a device tensor")


def make_cache(k_pool: torch.Tensor, v_pool: torch.Tensor, k_scale: float = 1.0,
               v_scale: float = 1.0) -> PaCache:
    """pa_cache for two [num_blocks][num_kv_heads][block_size][head_dim] pools.

    The scales are the dequantisation scales of an 8-bit (E4M3) cache: floats
    (one per pool), or device float32 tensors [num_kv_heads] (one per KV head,
    both pools alike); the other element types ignore float scales.
    """
    _require(k_pool.dim() == 4 and k_pool.shape == v_pool.shape and k_pool.dtype == v_pool.dtype,
             "k_pool and v_pool must be equal-shaped 4-D tensors")
    _require(k_pool.is_contiguous() and v_pool.is_contiguous(), "pools must be contiguous")
    _on_device(k_pool=k_pool, v_pool=v_pool)
    nb, hkv, bs, d = k_pool.shape
    per_head = isinstance(k_scale, torch.Tensor) or isinstance(v_scale, torch.Tensor)
    if not per_head:
        return PaCache(k_pool.data_ptr(), v_pool.data_ptr(), nb, hkv, bs, d, _dtype_code(k_pool),
                       float(k_scale), float(v_scale), None, None)
    for t in (k_scale, v_scale):
        _require(isinstance(t, torch.Tensor) and t.dtype == torch.float32 and t.is_contiguous()
                 and t.numel() == hkv and t.device.type != "cpu",
                 "per-head scales: contiguous device float32 tensors [num_kv_heads], both")
    return PaCache(k_pool.data_ptr(), v_pool.data_ptr(), nb, hkv, bs, d, _dtype_code(k_pool),
                   1.0, 1.0, k_scale.data_ptr(), v_scale.data_ptr())


def abi_version() -> int:
    return load().pa_abi_version()


def hip_runtime_version() -> int:
    return load().pa_hip_runtime_version()


def partials_bytes(num_seqs: int, num_heads: int, head_dim: int, max_parts: int) -> int:
    return load().pa_partials_bytes(num_seqs, num_heads, head_dim, max_parts)


def pa_kv_append(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None, k_scale=1.0,
                 v_scale=1.0) -> None:
    """Write k_new/v_new [n][Hkv][D] into the pools at slot_mapping (int64 [n]).

    For an 8-bit cache k_new/v_new are bf16 and are stored quantised with the
    pools' scales.
    """
    cache = make_cache(k_pool, v_pool, k_scale, v_scale)
    _on_device(k_new=k_new, v_new=v_new, slot_mapping=slot_mapping)
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous(),
             "slot_mapping must be contiguous int64")
    n = slot_mapping.numel()
    for t in (k_new, v_new):
        _require(t.dtype == _token_dtype(cache) and t.is_contiguous() and
                 tuple(t.shape) == (n, cache.num_kv_heads, cache.head_dim),
                 "k_new/v_new must be contiguous [n][num_kv_heads][head_dim] of the pool dtype "
                 "(bf16 for an 8-bit cache)")
    _check(load().pa_kv_append(ctypes.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                               n, _stream(stream)))


def pa_copy_blocks(k_pool, v_pool, block_pairs, stream=None) -> None:
    """Copy block src -> dst in both pools for each row of block_pairs (int64 [n][2])."""
    cache = make_cache(k_pool, v_pool, 1.0, 1.0)
    _on_device(block_pairs=block_pairs)
    _require(block_pairs.dtype == torch.int64 and block_pairs.is_contiguous() and
             (block_pairs.numel() == 0 or block_pairs.shape[-1] == 2),
             "block_pairs must be contiguous int64 [n][2]")
    _check(load().pa_copy_blocks(ctypes.byref(cache), _ptr(block_pairs), block_pairs.numel() // 2,
                                 _stream(stream)))


def pa_swap_blocks(k_pool, v_pool, host_k_pool, host_v_pool, block_pairs, direction: int,
                   stream=None, k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Whole-block copies between device pools and pinned host pools.

    ``direction`` PA_SWAP_OUT copies device block a to host block b for every
    row (a, b) of ``block_pairs`` (device int64 [n][2]); PA_SWAP_IN copies host
    block a to device block b.  The host pools are pinned CPU tensors shaped and
    typed like the device pools.
    """
    cache = make_cache(k_pool, v_pool, k_scale, v_scale)
    _require(host_k_pool.device.type == "cpu" and host_v_pool.device.type == "cpu" and
             host_k_pool.is_pinned() and host_v_pool.is_pinned(),
             "host pools must be pinned CPU tensors")
    _require(host_k_pool.shape[1:] == k_pool.shape[1:] and host_v_pool.shape == host_k_pool.shape
             and host_k_pool.dtype == k_pool.dtype and host_v_pool.dtype == k_pool.dtype and
             host_k_pool.is_contiguous() and host_v_pool.is_contiguous(),
             "host pools must be contiguous and match the device pools' block shape and type")
    _require(block_pairs.dtype == torch.int64 and block_pairs.is_contiguous() and
             block_pairs.device.type != "cpu" and
             (block_pairs.numel() == 0 or block_pairs.shape[-1] == 2),
             "block_pairs must be contiguous device int64 [n][2]")
    _check(load().pa_swap_blocks(ctypes.byref(cache), host_k_pool.data_ptr(),
                                 host_v_pool.data_ptr(), host_k_pool.shape[0], _ptr(block_pairs),
                                 block_pairs.numel() // 2, int(direction), _stream(stream)))


def decode_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int) -> int:
    """Bytes of workspace pa_decode needs on the current device, for any pools."""
    return load().pa_decode_workspace_bytes(num_seqs, num_heads, head_dim)


def decode_workspace_size(k_pool, v_pool, num_seqs: int, num_heads: int) -> int:
    """Bytes of workspace pa_decode needs for these pools on the current device."""
    cache = make_cache(k_pool, v_pool)
    return load().pa_decode_workspace_size(ctypes.byref(cache), num_seqs, num_heads)


def decode_workspace(num_seqs: int, num_heads: int, head_dim: int, device="cuda",
                     k_pool=None, v_pool=None) -> torch.Tensor:
    """A workspace for pa_decode (allocated through torch; contents irrelevant):
    sized exactly for the pools when they are given, else for any pools."""
    if k_pool is not None:
        n = decode_workspace_size(k_pool, v_pool if v_pool is not None else k_pool, num_seqs,
                                  num_heads)
    else:
        n = decode_workspace_bytes(num_seqs, num_heads, head_dim)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _decode_common(k_pool, v_pool, q, block_tables, context_lens, k_scale, v_scale):
    cache = make_cache(k_pool, v_pool, k_scale, v_scale)
    _on_device(q=q, block_tables=block_tables, context_lens=context_lens)
    _require(q.dim() == 3 and q.is_contiguous() and q.dtype == _token_dtype(cache) and
             q.shape[2] == cache.head_dim,
             "q must be contiguous [num_seqs][num_heads][head_dim] of the pool dtype "
             "(bf16 for an 8-bit cache)")
    num_seqs = q.shape[0]
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
             block_tables.is_contiguous() and block_tables.shape[0] == num_seqs,
             "block_tables must be contiguous int32 [num_seqs][max_blocks]")
    _require(context_lens.dtype == torch.int32 and context_lens.is_contiguous() and
             context_lens.numel() == num_seqs, "context_lens must be contiguous int32 [num_seqs]")
    return cache


def _variant(window, alibi_slopes, num_heads):
    """The pa_attn_variant argument: None (plain attention) or a reference to one."""
    if not window and alibi_slopes is None:
        return None
    if alibi_slopes is not None:
        _require(alibi_slopes.dtype == torch.float32 and alibi_slopes.is_contiguous() and
                 alibi_slopes.numel() == num_heads and alibi_slopes.device.type != "cpu",
                 "alibi_slopes must be a contiguous device float32 [num_heads]")
    return ctypes.byref(PaAttnVariant(int(window), 0, _ptr(alibi_slopes)))


def pa_decode(k_pool, v_pool, q, block_tables, context_lens, scale: float, out, workspace=None,
              stream=None, k_scale=1.0, v_scale=1.0, window: int = 0,
              alibi_slopes=None) -> None:
    """Decode attention into out [num_seqs][num_heads][head_dim].

    ``workspace`` (from decode_workspace()) enables the balanced split of the
    batch; None walks each sequence in one workgroup.  ``k_scale``/``v_scale``
    are an 8-bit cache's dequantisation scales.  ``window`` > 0 keeps only the
    last ``window`` positions; ``alibi_slopes`` (device float32 [num_heads])
    adds slope * (t - p) to the score of key t for the query at position p.
    """
    cache = _decode_common(k_pool, v_pool, q, block_tables, context_lens, k_scale, v_scale)
    num_seqs, num_heads = q.shape[0], q.shape[1]
    _require(out is not None and out.is_contiguous() and
             tuple(out.shape) == (num_seqs, num_heads, cache.head_dim),
             "out must be contiguous [num_seqs][num_heads][head_dim]")
    _on_device(out=out, workspace=workspace)
    ws_bytes = 0
    if workspace is not None:
        _require(workspace.is_contiguous(), "workspace must be contiguous")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().pa_decode(ctypes.byref(cache), _ptr(q), _ptr(block_tables), _ptr(context_lens),
                            num_seqs, num_heads, block_tables.shape[1], float(scale),
                            _variant(window, alibi_slopes, num_heads), _ptr(out),
                            _dtype_code(out), _ptr(workspace), ws_bytes, _stream(stream)))


def pa_decode_static(k_pool, v_pool, q, block_tables, context_lens, scale: float, out,
                     stream=None, k_scale=1.0, v_scale=1.0, window: int = 0,
                     alibi_slopes=None) -> None:
    """pa_decode's balanced split over the library's own device scratch (no
    workspace argument, nothing allocated); see include/pagedattn.h."""
    cache = _decode_common(k_pool, v_pool, q, block_tables, context_lens, k_scale, v_scale)
    num_seqs, num_heads = q.shape[0], q.shape[1]
    _require(out is not None and out.is_contiguous() and
             tuple(out.shape) == (num_seqs, num_heads, cache.head_dim),
             "out must be contiguous [num_seqs][num_heads][head_dim]")
    _on_device(out=out)
    _check(load().pa_decode_static(ctypes.byref(cache), _ptr(q), _ptr(block_tables),
                                   _ptr(context_lens), num_seqs, num_heads,
                                   block_tables.shape[1], float(scale),
                                   _variant(window, alibi_slopes, num_heads), _ptr(out),
                                   _dtype_code(out), _stream(stream)))


def pa_decode_append(k_pool, v_pool, q, k_new, v_new, block_tables, context_lens, scale: float,
                     out, workspace=None, stream=None, k_scale=1.0, v_scale=1.0, window: int = 0,
                     alibi_slopes=None) -> None:
    """Append every sequence's new K/V at position L_i - 1 and decode, in one launch.

    ``k_new``/``v_new``: [num_seqs][num_kv_heads][head_dim] of the token dtype
    (bf16 for an 8-bit cache).  Same result as pa_kv_append with the
    table-derived slots followed by pa_decode.
    """
    cache = _decode_common(k_pool, v_pool, q, block_tables, context_lens, k_scale, v_scale)
    num_seqs, num_heads = q.shape[0], q.shape[1]
    _on_device(k_new=k_new, v_new=v_new)
    for t in (k_new, v_new):
        _require(t is not None and t.is_contiguous() and t.dtype == _token_dtype(cache) and
                 tuple(t.shape) == (num_seqs, cache.num_kv_heads, cache.head_dim),
                 "k_new/v_new must be contiguous [num_seqs][num_kv_heads][head_dim] of the "
                 "token dtype")
    _require(out is not None and out.is_contiguous() and
             tuple(out.shape) == (num_seqs, num_heads, cache.head_dim),
             "out must be contiguous [num_seqs][num_heads][head_dim]")
    _on_device(out=out, workspace=workspace)
    ws_bytes = 0
    if workspace is not None:
        _require(workspace.is_contiguous(), "workspace must be contiguous")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().pa_decode_append(ctypes.byref(cache), _ptr(q), _ptr(k_new), _ptr(v_new),
                                   _ptr(block_tables), _ptr(context_lens), num_seqs, num_heads,
                                   block_tables.shape[1], float(scale),
                                   _variant(window, alibi_slopes, num_heads), _ptr(out),
                                   _dtype_code(out), _ptr(workspace), ws_bytes,
                                   _stream(stream)))


def pa_decode_partitions(k_pool, v_pool, q, block_tables, context_lens, scale: float,
                         partition_size: int, part_out, part_max, part_sum, stream=None,
                         k_scale=1.0, v_scale=1.0) -> None:
    """Split-KV decode partials; see include/pagedattn.h."""
    cache = _decode_common(k_pool, v_pool, q, block_tables, context_lens, k_scale, v_scale)
    num_seqs, num_heads = q.shape[0], q.shape[1]
    _require(part_out is not None and part_out.dim() == 4 and part_out.is_contiguous() and
             part_out.dtype == torch.float32 and
             tuple(part_out.shape[:2]) == (num_seqs, num_heads) and
             part_out.shape[3] == cache.head_dim,
             "part_out must be contiguous float32 [num_seqs][num_heads][max_parts][head_dim]")
    max_parts = part_out.shape[2]
    for t in (part_max, part_sum):
        _require(t is not None and t.dtype == torch.float32 and t.is_contiguous() and
                 tuple(t.shape) == (num_seqs, num_heads, max_parts),
                 "part_max/part_sum must be contiguous float32 [num_seqs][num_heads][max_parts]")
    _on_device(part_out=part_out, part_max=part_max, part_sum=part_sum)
    _check(load().pa_decode_partitions(ctypes.byref(cache), _ptr(q), _ptr(block_tables),
                                       _ptr(context_lens), num_seqs, num_heads,
                                       block_tables.shape[1], float(scale), int(partition_size),
                                       _ptr(part_out), _ptr(part_max), _ptr(part_sum), max_parts,
                                       _stream(stream)))


def prefill_workspace_bytes(num_seqs: int, num_tokens: int, num_heads: int,
                            num_kv_heads: int) -> int:
    return load().pa_prefill_workspace_bytes(num_seqs, num_tokens, num_heads, num_kv_heads)


def prefill_workspace(num_seqs: int, num_tokens: int, num_heads: int, num_kv_heads: int,
                      device="cuda") -> torch.Tensor:
    """A device workspace for pa_prefill (256-byte aligned, as torch allocates)."""
    n = max(prefill_workspace_bytes(num_seqs, num_tokens, num_heads, num_kv_heads), 16)
    return torch.empty(n, dtype=torch.uint8, device=device)


def pa_prefill(k_pool, v_pool, q, block_tables, query_start, context_lens, scale: float, out,
               workspace=None, stream=None, k_scale: float = 1.0, v_scale: float = 1.0,
               window: int = 0, alibi_slopes=None) -> None:
    """Causal attention of a flattened mixed batch (see include/pagedattn.h).

    ``window`` > 0 restricts each query to its last ``window`` positions;
    ``alibi_slopes`` (device float32 [num_heads]) adds slope * (t - p) to scores.
    """
    cache = make_cache(k_pool, v_pool, k_scale, v_scale)
    _on_device(q=q, out=out, block_tables=block_tables, query_start=query_start,
               context_lens=context_lens, workspace=workspace)
    _require(q.dtype == torch.bfloat16 and q.is_contiguous() and q.dim() == 3 and
             q.shape[2] == cache.head_dim,
             "q must be contiguous bf16 [num_tokens][num_heads][head_dim] with the pools' "
             "head_dim")
    num_tokens, num_heads = q.shape[0], q.shape[1]
    _require(context_lens.dtype == torch.int32 and context_lens.dim() == 1 and
             context_lens.is_contiguous(), "context_lens must be contiguous int32 [num_seqs]")
    num_seqs = context_lens.shape[0]
    _require(out is not None and out.shape == q.shape and out.is_contiguous() and
             out.dtype in (torch.float32, torch.bfloat16),
             "out must be contiguous float32 or bfloat16 of q's shape")
    _require(block_tables.dtype == torch.int32 and block_tables.is_contiguous() and
             block_tables.dim() == 2 and block_tables.shape[0] == num_seqs,
             "block_tables must be contiguous int32 [num_seqs][max_blocks]")
    _require(query_start.dtype == torch.int32 and query_start.is_contiguous() and
             query_start.numel() == num_seqs + 1,
             "query_start must be contiguous int32 [num_seqs + 1]")
    if workspace is None:
        workspace = prefill_workspace(num_seqs, num_tokens, num_heads, k_pool.shape[1],
                                      device=q.device)
    _require(workspace.is_contiguous(), "workspace must be contiguous")
    variant = _variant(window, alibi_slopes, num_heads)
    _check(load().pa_prefill(ctypes.byref(cache), _ptr(q), _ptr(block_tables), _ptr(query_start),
                             _ptr(context_lens), num_seqs, num_tokens, num_heads,
                             block_tables.shape[1], float(scale), variant, _ptr(out),
                             _dtype_code(out),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream)))


def pa_splitkv_reduce(part_out, part_max, part_sum, context_lens, partition_size: int, out,
                      lse=None, stream=None) -> None:
    """Merge split-KV partials into out [num_seqs][num_heads][head_dim]."""
    _require(part_out.dim() == 4 and part_out.dtype == torch.float32 and part_out.is_contiguous(),
             "part_out must be contiguous float32 [num_seqs][num_heads][max_parts][head_dim]")
    num_seqs, num_heads, max_parts, head_dim = part_out.shape
    for t in (part_max, part_sum):
        _require(t.dtype == torch.float32 and t.is_contiguous() and
                 tuple(t.shape) == (num_seqs, num_heads, max_parts),
                 "part_max/part_sum must be contiguous float32 [num_seqs][num_heads][max_parts]")
    _require(context_lens.dtype == torch.int32 and context_lens.numel() == num_seqs,
             "context_lens must be int32 [num_seqs]")
    _require(out.is_contiguous() and tuple(out.shape) == (num_seqs, num_heads, head_dim),
             "out must be contiguous [num_seqs][num_heads][head_dim]")
    _require(context_lens.is_contiguous(), "context_lens must be contiguous")
    _on_device(part_out=part_out, part_max=part_max, part_sum=part_sum,
               context_lens=context_lens, out=out, lse=lse)
    if lse is not None:
        _require(lse.dtype == torch.float32 and lse.is_contiguous() and
                 tuple(lse.shape) == (num_seqs, num_heads), "lse must be float32 [num_seqs][num_heads]")
    _check(load().pa_splitkv_reduce(_ptr(part_out), _ptr(part_max), _ptr(part_sum),
                                    _ptr(context_lens), num_seqs, num_heads, head_dim, max_parts,
                                    int(partition_size), _ptr(out), _dtype_code(out), _ptr(lse),
                                    _stream(stream)))


# ---------------------------------------------------------------------------
# block manager (host only)
# ---------------------------------------------------------------------------

REQUEST_STATES = {0: "waiting", 1: "running", 2: "swapped"}
PREEMPT_MODES = {"recompute": 0, "swap": 1}


class StepPlan:
    """One step's plan as numpy arrays (copied out of the manager)."""

    def __init__(self, p: PaStepPlan):
        import numpy as np

        def arr(ptr, n, dtype):
            if n == 0:
                return np.zeros(0, dtype=dtype)
            nbytes = n * np.dtype(dtype).itemsize
            return np.frombuffer(ctypes.string_at(ptr, nbytes), dtype=dtype).copy()

        S = p.num_seqs
        self.seq_ids = arr(p.seq_ids, S, np.int64)
        self.query_start = arr(p.query_start, S + 1, np.int32)
        self.context_lens = arr(p.context_lens, S, np.int32)
        self.slot_mapping = arr(p.slot_mapping, p.num_tokens, np.int64)
        self.max_blocks = p.max_blocks
        self.block_tables = arr(p.block_tables, S * p.max_blocks, np.int32).reshape(S, p.max_blocks)
        self.cow_pairs = arr(p.cow_pairs, 2 * p.num_cow, np.int64).reshape(-1, 2)
        self.swap_out = arr(p.swap_out_pairs, 2 * p.num_swap_out, np.int64).reshape(-1, 2)
        self.swap_in = arr(p.swap_in_pairs, 2 * p.num_swap_in, np.int64).reshape(-1, 2)
        modes = {v: k for k, v in PREEMPT_MODES.items()}
        self.preempted = list(zip(arr(p.preempted_ids, p.num_preempted, np.int64).tolist(),
                                  [modes[m] for m in arr(p.preempted_modes, p.num_preempted,
                                                         np.int32).tolist()]))


class BlockManager:
    """The native block manager (include/pa_block_manager.h) behind a Python object."""

    def __init__(self, num_gpu_blocks: int, num_cpu_blocks: int, block_size: int,
                 prefix_caching: bool = True, preempt_mode: str = "recompute",
                 watermark_blocks: int = 0):
        _require(preempt_mode in PREEMPT_MODES, "preempt_mode is 'recompute' or 'swap'")
        cfg = PaBmConfig(num_gpu_blocks, num_cpu_blocks, block_size, int(bool(prefix_caching)),
                         PREEMPT_MODES[preempt_mode], watermark_blocks)
        handle = _vp()
        self._h = None
        _check(load().pa_bm_create(ctypes.byref(cfg), ctypes.byref(handle)))
        self._h = handle
        self.B = block_size
        self.num_gpu_blocks = num_gpu_blocks
        self.num_cpu_blocks = num_cpu_blocks

    def __del__(self):
        if getattr(self, "_h", None) is not None and _lib is not None:
            _lib.pa_bm_destroy(self._h)
            self._h = None

    @staticmethod
    def _tokens(tokens):
        import numpy as np

        a = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        _require(a.ndim == 1 and (a.size == 0 or (a.min() >= -2**31 and a.max() < 2**31)),
                 "tokens must be a 1-D sequence of int32 values")
        return np.ascontiguousarray(a.astype(np.int32))

    def add_request(self, rid: int, tokens) -> None:
        t = self._tokens(tokens)
        _check(load().pa_bm_add_request(self._h, int(rid), t.ctypes.data, t.size))

    def append_token(self, rid: int, token: int) -> None:
        self.append_tokens(rid, [token])

    def append_tokens(self, rid: int, tokens) -> None:
        t = self._tokens(tokens)
        _check(load().pa_bm_append_tokens(self._h, int(rid), t.ctypes.data, t.size))

    def append_batch(self, rids, tokens) -> None:
        """Appends tokens[i] to request rids[i] for every i, in one call."""
        import numpy as np

        r = np.ascontiguousarray(np.asarray(rids, dtype=np.int64))
        t = self._tokens(tokens)
        _require(r.ndim == 1 and r.size == t.size, "rids and tokens must be equal-length 1-D")
        _check(load().pa_bm_append_batch(self._h, r.ctypes.data, t.ctypes.data, r.size))

    def fork(self, parent: int, child: int) -> None:
        _check(load().pa_bm_fork(self._h, int(parent), int(child)))

    def finish(self, rid: int) -> None:
        _check(load().pa_bm_finish(self._h, int(rid)))

    def schedule(self, token_budget: int) -> StepPlan:
        p = PaStepPlan()
        _check(load().pa_bm_schedule(self._h, int(token_budget), ctypes.byref(p)))
        return StepPlan(p)

    def stats(self) -> dict:
        st = PaBmStats()
        _check(load().pa_bm_get_stats(self._h, ctypes.byref(st)))
        return {name: getattr(st, name) for name in _BM_STATS}

    def request_info(self, rid: int) -> dict:
        info = PaRequestInfo()
        _check(load().pa_bm_request_info(self._h, int(rid), ctypes.byref(info)))
        return dict(state=REQUEST_STATES[info.state], computed=info.computed,
                    num_tokens=info.num_tokens, arrival=info.arrival,
                    num_blocks=info.num_blocks, num_cpu_blocks=info.num_cpu_blocks)

    def _ids(self, fn, *args) -> list:
        import numpy as np

        count = _i64()
        fn(self._h, *args, None, 0, ctypes.byref(count))
        out = np.zeros(max(count.value, 1), dtype=np.int32)
        _check(fn(self._h, *args, out.ctypes.data, out.size, ctypes.byref(count)))
        return out[:count.value].tolist()

    def table(self, rid: int) -> list:
        return self._ids(load().pa_bm_blocks, int(rid), 0)

    def cpu_blocks(self, rid: int) -> list:
        return self._ids(load().pa_bm_blocks, int(rid), 1)

    def free_list(self, cpu: bool = False) -> list:
        return self._ids(load().pa_bm_free_list, int(bool(cpu)))

    def refcounts(self) -> list:
        import numpy as np

        out = np.zeros(self.num_gpu_blocks, dtype=np.int32)
        _check(load().pa_bm_refcounts(self._h, out.ctypes.data, out.size))
        return out.tolist()


def probe_stream_read(src: torch.Tensor, workgroups: int, sink: torch.Tensor,
                      xcd_mask: int = 0xFF, stream=None) -> None:
    """Read all of src (device, contiguous, a multiple of 64 KiB) once with
    the streaming-read probe; sink receives 16 bytes per workgroup."""
    _on_device(src=src, sink=sink)
    _require(src.is_contiguous() and sink.is_contiguous() and
             sink.numel() * sink.element_size() >= 16 * workgroups,
             "src contiguous; sink contiguous with 16 bytes per workgroup")
    _check(load().pa_probe_stream_read(_ptr(src), src.numel() * src.element_size(),
                                       int(workgroups), int(xcd_mask), _ptr(sink),
                                       _stream(stream)))


def raw_call(name: str, *args) -> int:
    """Call an entry point with raw arguments and return its status (for ABI tests)."""
    return getattr(load(), name)(*args)
