"""Float64 CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``paged_kv_cache_24_amd``) never imports it and shares no code,
header, table or helper with it.

Every function follows a passage of the source pages; each docstring cites the
page title and section it restates.
"""

from .paged_attention import (  # noqa: F401
    bits_to_float64,
    kv_bytes_per_token,
    ref_reshape_and_cache,
    ref_copy_blocks,
    gather_tokens,
    ref_contiguous_attention,
    ref_decode,
    ref_decode_one,
    ref_decode_multi,
    ref_prefill_paged,
    ref_prefill_rows,
    ref_partition_state,
    ref_merge_partitions,
)
from .kv_fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_to_float64,
    float_to_e4m3,
    quantize_e4m3_rows,
    dequantize_e4m3_rows,
    ref_reshape_and_cache_fp8,
    gather_scales,
    ref_decode_fp8,
    ref_prefill_rows_fp8,
    ref_prefill_paged_fp8,
)
