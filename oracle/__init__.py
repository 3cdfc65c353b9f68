"""CPU oracle for paged attention decode.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package. The HIP library never imports it, and
nothing here imports the HIP library or its Python binding.

Attention is plain NumPy in float64 (``paged_attention.py``); the block
manager and its per-step scheduler are plain Python (``block_manager.py``).
Each module lists the passages it follows.
"""

from .paged_attention import (  # noqa: F401
    E4M3_MAX,
    alibi_bias,
    alibi_slopes,
    attended_range,
    blocks_needed,
    copy_blocks,
    decode,
    decode_partitions,
    e4m3_value,
    fp8_encode,
    fp8_quantize,
    fp8_to_f64,
    gather_rows,
    kv_append,
    last_block_waste,
    prefill,
    query_position,
    slot_of,
    splitkv_merge,
    to_f64,
    visible_keys,
)
